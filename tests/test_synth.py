"""The seeded generators: reproducible, the documented shapes and distributions."""
import math

import numpy as np

import synth


def test_reproducible_and_layer_dependent():
    wl = synth.WORKLOADS["tiny"]
    a = synth.make_layer_inputs(wl, 0, layer=0)
    b = synth.make_layer_inputs(wl, 0, layer=0)
    c = synth.make_layer_inputs(wl, 0, layer=1)
    for key in ["q_s", "k_s", "w", "v_r"]:
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_shapes_and_planted_keys():
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_layer_inputs(wl, 1)
    H, T, d = wl.H_s, 256, wl.d
    assert x["q_s"].shape == (H, T, d) and x["k_s"].shape == (H, T, d)
    assert x["w"].shape == (wl.H_r, H) and x["v_r"].shape == (T, wl.H_kv, d)
    assert np.allclose(x["w"].sum(axis=1), 1.0, atol=1e-6) and np.all(x["w"] >= 0)
    hot = x["hot_tokens"]
    assert hot[0] == 0 and len(hot) == 1 + round(0.01 * T)
    # the boost a*u_h = 0.75 sqrt(d) u_h shows up in the mean key of the hot tokens
    cold = np.setdiff1d(np.arange(T), hot)
    gap = np.linalg.norm(x["k_s"][:, hot].mean(axis=1) - x["k_s"][:, cold].mean(axis=1), axis=1)
    assert np.all(np.abs(gap - 0.75 * math.sqrt(d)) < 2.5)


def test_bf16_inputs_are_bf16_values():
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 0, lengths=[300], H_s=2, H_r=3, H_kv=1, d=32)
    for key in ["q_s", "k_s", "v_r"]:
        v = x[key]
        assert np.array_equal(synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(v)), v)


def test_varlen_lengths_and_page_table():
    wl = synth.WORKLOADS["varlen_14b8b"]
    lens = synth.make_lengths(wl, 0)
    assert len(lens) == 16 and all(1024 <= n <= 16384 for n in lens)
    table, n_pages = synth.make_page_table(lens, 16, seed=0)
    used = table[table >= 0]
    assert n_pages == sum((n + 15) // 16 for n in lens)
    assert np.array_equal(np.sort(used), np.arange(n_pages))
