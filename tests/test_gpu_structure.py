"""GPU checks of the fused retrieve against what the mathematics fixes, beside the element-wise
oracle comparisons of test_gpu_parity.py:

* a V whose rows are all equal to v gives O = v for every query row, whatever the kept blocks
  and the mixing weights (the renormalised mixed rows sum to one);
* a "read-out" V, V[kv, j0 + c, c] = 1 and 0 elsewhere, makes O[., g, c] equal the renormalised
  mixed map of receiver head g at key j0 + c, so the on-chip mixed map itself is compared with
  the oracle's (not only its products with V);
* permuting the sender heads (Q, K and the columns of W together) leaves the output unchanged up
  to rounding: the GPU's head mix depends on the heads only through W;
* weights that bf16 cannot hold (the mix multiplies the bf16 probabilities by a bf16 hi part and
  a bf16 lo part of each weight) still enter the read-out mixed map to fp16 precision, whichever
  path the receiver's heads take and whichever head chunk the weight falls in.

Also the retrieve's work order that a store carries: a permutation of its block rows, dealt to
the XCDs as the header describes it.

[MapFlow开源, section 算得省的:融合内核执行]: the kernel mixes the sender heads linearly on chip,
renormalises the rows and multiplies by the receiver's own V.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_out_close, gpu_store_for_oracle, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mf():
    import cross_model_attention_amd as m
    return m


def _case(seed, lengths, H_s=32, H_r=24, H_kv=8, d=128):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, seed, lengths=lengths, H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
    return wl, x, float(np.float32(wl.tau))


def _compress(mf, x, tau, B):
    store = mf.compress(to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16"), tau, B, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return store


@pytest.mark.parametrize("lengths,heads", [([300, 77], (32, 24, 8, 128)), ([200], (40, 32, 8, 64))])
def test_constant_v_gives_that_row(mf, lengths, heads):
    wl, x, tau = _case(41, lengths, *heads)
    say(f"case: constant V lengths={lengths} heads={heads}")
    store = _compress(mf, x, tau, wl.B)
    T, H_kv, d = x["T"], x["H_kv"], x["d"]
    v = synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(
        np.random.default_rng(41).standard_normal((H_kv, d)).astype(np.float32)))
    V = np.broadcast_to(v[None], (T, H_kv, d)).copy()
    O = mf.retrieve(store, to_dev(x["w"]), to_dev(V, "bf16"), x["kv_head_map"])
    torch.cuda.synchronize()
    want = np.broadcast_to(v[np.asarray(x["kv_head_map"])][None], O.shape)
    assert_out_close(O.cpu().numpy(), want, "O_r with constant V")


@pytest.mark.parametrize("j0", [0, 64])
def test_v_readout_exposes_the_mixed_map(mf, j0):
    wl, x, tau = _case(42, [330, 150])
    say(f"case: V read-out j0={j0}")
    store = _compress(mf, x, tau, wl.B)
    host = store.to_host()
    T, H_kv, d, cu = x["T"], x["H_kv"], x["d"], x["cu_seqlens"]
    V = np.zeros((T, H_kv, d), dtype=np.float32)
    for s in range(len(cu) - 1):
        for c in range(d):
            j = j0 + c
            if j < cu[s + 1] - cu[s]:
                V[cu[s] + j, :, c] = 1.0
    O = mf.retrieve(store, to_dev(x["w"]), to_dev(V, "bf16"), x["kv_head_map"])
    torch.cuda.synchronize()
    got = O.cpu().numpy().astype(np.float64)
    want = oracle.retrieve(gpu_store_for_oracle(host, cu, wl.B, x["H_s"]), x["w"], V, x["kv_head_map"])
    assert_out_close(got, want, "read-out of the mixed map")
    # a renormalised mixed map with Dirichlet (non-negative) weights lies in [0, 1]
    assert got.min() >= -1e-3 and got.max() <= 1 + 1e-3


def test_sender_head_permutation_invariance(mf):
    wl, x, tau = _case(43, [280, 96])
    say("case: sender-head permutation")
    perm = np.random.default_rng(43).permutation(x["H_s"])
    store = _compress(mf, x, tau, wl.B)
    xp = dict(x, q_s=np.ascontiguousarray(x["q_s"][perm]), k_s=np.ascontiguousarray(x["k_s"][perm]),
              w=np.ascontiguousarray(x["w"][:, perm]))
    store_p = _compress(mf, xp, tau, wl.B)
    h, hp = store.to_host(), store_p.to_host()
    # the head-summed masses only change in rounding order: the same blocks are kept
    assert np.array_equal(h["block_ptr"], hp["block_ptr"]) and np.array_equal(h["block_idx"], hp["block_idx"])
    assert np.array_equal(h["probs"][:, perm], hp["probs"]), "stored values move with their heads"
    V = to_dev(x["v_r"], "bf16")
    O = mf.retrieve(store, to_dev(x["w"]), V, x["kv_head_map"])
    Op = mf.retrieve(store_p, to_dev(xp["w"]), V, x["kv_head_map"])
    torch.cuda.synchronize()
    assert_out_close(Op.cpu().numpy(), O.cpu().numpy().astype(np.float64), "O_r with permuted sender heads")
    assert_out_close(Op.cpu().numpy(),
                     oracle.retrieve(gpu_store_for_oracle(h, x["cu_seqlens"], wl.B, x["H_s"]), x["w"], x["v_r"],
                                     x["kv_head_map"]), "O_r (permuted) vs the oracle")


# (H_s, H_r, H_kv, d): 8 heads of one KV group (one head per wave), 32 heads in KV groups of 4
# (the half-block path), 16 heads in KV groups of 4 with a last chunk of two 8-head groups, and 13
# heads of 13 KV groups (no two heads of a wave share V: the general path)
@pytest.mark.parametrize("heads", [(40, 8, 1, 128), (40, 32, 8, 128), (44, 16, 4, 64), (44, 13, 13, 128)])
def test_mix_keeps_the_weights_low_bits(mf, heads):
    H_s, H_r, H_kv, d = heads
    wl, x, tau = _case(44, [300, 90], H_s, H_r, H_kv, d)
    say(f"case: low weight bits heads={heads}")
    store = _compress(mf, x, tau, wl.B)
    host = store.to_host()
    # receiver head g mixes sender head g mod 32 with weight 1/2 + 2^-10 and sender head
    # 32 + g mod (H_s - 32) (in the last chunk) with weight 1 + 2^-8 + 2^-12: bf16 rounds them to
    # 1/2 and 1 + 2^-7, relative errors 2e-3 and 3.7e-3, eight times the fp16 rounding of the map
    W = np.zeros((H_r, H_s), dtype=np.float32)
    for g in range(H_r):
        W[g, g % 32] = 0.5 + 2.0 ** -10
        W[g, 32 + g % (H_s - 32)] = 1.0 + 2.0 ** -8 + 2.0 ** -12
    T, cu, j0 = x["T"], x["cu_seqlens"], 64
    V = np.zeros((T, H_kv, d), dtype=np.float32)
    for s in range(len(cu) - 1):
        for c in range(d):
            if j0 + c < cu[s + 1] - cu[s]:
                V[cu[s] + j0 + c, :, c] = 1.0
    O = mf.retrieve(store, to_dev(W), to_dev(V, "bf16"), x["kv_head_map"])
    torch.cuda.synchronize()
    got = O.cpu().numpy().astype(np.float64)
    want = oracle.retrieve(gpu_store_for_oracle(host, cu, wl.B, H_s), W, V, x["kv_head_map"])
    # each read-out value is one fp16-rounded mixed-map element over an fp32 denominator: within
    # 2^-11 relative (half an fp16 ulp) plus fp32 rounding
    err = np.abs(got - want)
    bound = 5.2e-4 * np.abs(want) + 1e-9
    assert np.count_nonzero(want) > 1000
    assert np.all(err <= bound), f"worst relative error {float((err / (np.abs(want) + 1e-30)).max()):.3e}"


def _documented_work_order(lengths, B):
    """The retrieve's work order as the header states it: block rows by descending in-sequence
    index (ties in row order), then in each whole run of 64 entries XCD x (entry p runs on XCD
    p mod 8) takes 8 consecutive entries of that order, the x-th group of 8 in even runs and the
    (7 - x)-th in odd runs; a last partial run keeps the sorted order."""
    I = [i for n in lengths for i in range(-(-n // B))]
    srt = sorted(range(len(I)), key=lambda b: -I[b])
    o = list(srt)
    for run, m in enumerate(range(0, len(srt) - 63, 64)):
        for x in range(8):
            src = 7 - x if run & 1 else x
            for k in range(8):
                o[m + 8 * k + x] = srt[m + 8 * src + k]
    return np.array(o, np.int32)


@pytest.mark.parametrize("lengths", [[64 * 200 + 17], [3000, 64 * 150, 900, 5000], [50]])
def test_retrieve_work_order_is_the_documented_deal(mf, lengths):
    import ctypes
    from cross_model_attention_amd import mapflow as mfm

    B, H_s, d = 64, 8, 64
    T = sum(lengths)
    g = torch.Generator(device="cuda").manual_seed(5)
    Q = torch.randn(H_s, T, d, device="cuda", generator=g).to(torch.bfloat16)
    K = torch.randn(H_s, T, d, device="cuda", generator=g).to(torch.bfloat16)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    store = mf.compress(Q, K, 0.9, B, cu_seqlens=cu)
    r = store.raw
    want = _documented_work_order(lengths, B)
    assert r.n_order == r.n_brow == len(want)
    # the store's order array, copied out by the library's own 16-byte copy kernel
    nbytes = -(-r.n_order * 4 // 16) * 16
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    mfm.check(mfm._L.mf_copy_probe(store.ctx.handle, ctypes.c_void_p(dst.data_ptr()),
                                   ctypes.c_void_p(r.brow_order), nbytes, mfm._stream(None)))
    got = dst.cpu().numpy()[: r.n_order]
    say(f"work order of {lengths}: {r.n_order} rows, first 16 {got[:16].tolist()}")
    assert sorted(got.tolist()) == list(range(r.n_brow)), "not a permutation of the block rows"
    np.testing.assert_array_equal(got, want)
