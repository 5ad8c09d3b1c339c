"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element, on
seeded inputs small enough for the oracle to finish in seconds but spanning several tiles and a
ragged tail.  Edge cases: single partial block, one-token sequences, tau = 1, forced-only
selection, varlen with an empty sequence, paged V."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_out_close, brow_table, check_selection, dense_maps, gpu_store_for_oracle, say,
                    sets_agree, to_dev, ulp_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mf():
    import cross_model_attention_amd as m
    return m


def _f32(x):
    return float(np.float32(x))


def _compress_case(mf, x, tau, B, dtype):
    say(f"case: compress T={x['T']} H_s={x['H_s']} d={x['d']} B={B} tau={tau} lengths={x['lengths'][:6]}")
    Q, K = to_dev(x["q_s"], dtype), to_dev(x["k_s"], dtype)
    store = mf.compress(Q, K, tau, B, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return store, store.to_host()


def _check_compress(x, host, ref, tau, B):
    cu = x["cu_seqlens"]
    rows = brow_table(cu, B)
    assert host["block_ptr"].shape[0] == len(rows) + 1
    maps = dense_maps(x["q_s"], x["k_s"], cu)
    excused = 0
    for b, (s, I) in enumerate(rows):
        got = host["block_idx"][host["block_ptr"][b]:host["block_ptr"][b + 1]].tolist()
        assert got == sorted(got) and len(set(got)) == len(got)
        ok, why = sets_agree(got, ref.rows[b], tau)
        assert ok, f"block row {b} (seq {s}, I={I}): {why}; gpu {got} oracle {ref.rows[b]['kept']}"
        excused += bool(why)
        n = int(cu[s + 1] - cu[s])
        r0 = I * B
        rows_b = min(n, r0 + B) - r0
        for t in range(host["block_ptr"][b], host["block_ptr"][b + 1]):
            J = int(host["block_idx"][t])
            p = host["probs"][t]
            for h in range(x["H_s"]):
                A = np.zeros((B, B))
                c1 = min(n, (J + 1) * B)
                A[:rows_b, : c1 - J * B] = maps[s][h][r0:r0 + rows_b, J * B:c1]
                err = np.abs(p[h] - A)
                assert np.all(err <= ulp_bf16(A) + 1e-6), \
                    f"probs block ({I},{J}) head {h}: max excess {(err - ulp_bf16(A)).max():.3e}"
    # kept row mass equals the sum of the stored probabilities of each row (fp32 accumulation)
    rkm = host["row_kept_mass"]
    for b, (s, I) in enumerate(rows):
        n = int(cu[s + 1] - cu[s])
        tok0 = int(cu[s]) + I * B
        rows_b = min(n, I * B + B) - I * B
        lo, hi = host["block_ptr"][b], host["block_ptr"][b + 1]
        want = host["probs"][lo:hi, :, :rows_b, :].sum(axis=(0, 3))       # [H_s, rows]
        assert np.allclose(rkm[:, tok0:tok0 + rows_b], want, rtol=1e-6, atol=1e-7)
        if sorted(ref.rows[b]["kept"]) == host["block_idx"][lo:hi].tolist():
            # each stored value may sit one bf16 ulp from the oracle's rounding of the same entry
            r_or = ref.rows[b]
            slack = sum(ulp_bf16(r_or["probs"][J][:, :rows_b, :]).sum(axis=2) for J in r_or["kept"])
            assert np.all(np.abs(rkm[:, tok0:tok0 + rows_b] - r_or["row_kept_mass"]) <= slack + 1e-6)
    return excused


@pytest.mark.parametrize("k", range(16))
def test_compress_random_shapes(mf, k):
    """A seeded sweep of compress shapes (B 32 or 64, d 64 or 128, 1..64 sender heads, bf16 or
    fp32 inputs, tau in [0.5, 1], 1..3 ragged sequences) through the oracle's compress checks:
    kept sets (ties excused), probabilities within one bf16 ulp + 1e-6 of the exact map, kept
    row mass."""
    r = np.random.default_rng(np.random.SeedSequence([4343, k]))
    B = int(r.choice([32, 64]))
    d = int(r.choice([64, 128]))
    H_s = int(r.integers(1, 65))
    dtype = str(r.choice(["bf16", "f32"]))
    tau = _f32(r.uniform(0.5, 1.0))
    lengths = [int(n) for n in r.integers(1, 3 * B + 40, size=int(r.integers(1, 4)))]
    wl = synth.WORKLOADS["tiny" if dtype == "f32" else "pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 500 + k, lengths=lengths, H_s=H_s, H_r=2, H_kv=1, d=d)
    store, host = _compress_case(mf, x, tau, B, dtype)
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    _check_compress(x, host, ref, tau, B)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_compress_tiny_fp32(mf, seed):
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_layer_inputs(wl, seed)
    tau = _f32(wl.tau)
    store, host = _compress_case(mf, x, tau, wl.B, "f32")
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
    ex = _check_compress(x, host, ref, tau, wl.B)
    say(f"  nnzb gpu={host['nnzb']} oracle={len(ref.block_idx)} excused rows={ex}")


@pytest.mark.parametrize("lengths,H_s,d,B,tau,seed", [
    ([357], 32, 128, 64, 0.95, 0),           # 8B->3B shapes, ragged tail
    ([200, 64, 1, 130], 8, 64, 32, 0.9, 1),  # varlen incl. a one-token sequence
    ([50], 40, 128, 64, 0.95, 2),            # single partial block, 40 heads
    ([300], 16, 128, 64, 1.0, 3),            # tau = 1: every causal block
    ([260, 0, 99], 8, 128, 32, 0.05, 4),     # forced blocks only; an empty sequence
])
def test_compress_bf16_shapes(mf, lengths, H_s, d, B, tau, seed):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, seed, lengths=lengths, H_s=H_s, H_r=8, H_kv=2, d=d)
    tau = _f32(tau)
    store, host = _compress_case(mf, x, tau, B, "bf16")
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    _check_compress(x, host, ref, tau, B)
    if tau >= 1.0:
        n_causal = sum(((n + B - 1) // B) * ((n + B - 1) // B + 1) // 2 for n in lengths)
        assert host["nnzb"] == n_causal


def test_compress_rows_spanning_several_gather_items(mf):
    # tau = 1 keeps every causal block, so the last block rows of a 4200-token sequence at B = 32
    # hold up to 132 kept blocks: more than one gather work item (128 kept blocks), with a short
    # remainder.  Their probabilities and kept row mass are compared with the oracle.
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 5, lengths=[4200], H_s=4, H_r=4, H_kv=2, d=64)
    tau = _f32(1.0)
    B = 32
    store, host = _compress_case(mf, x, tau, B, "bf16")
    counts = np.diff(host["block_ptr"])
    assert counts.max() == 132 and (counts > 128).sum() == 4
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    _check_compress(x, host, ref, tau, B)


def test_compress_scores_far_above_the_running_maximum(mf):
    """Block statistics past a row's first block are summed against the row's running maximum;
    when a later block's scores sit far above it (z would reach 2^64) the wave redoes the block
    with the block maximum.  Keys of block 1 are copies of queries of block rows 2 and 3 scaled by
    4 (exact in bf16), so those rows' scores in block 1 exceed everything before them by ~2^65."""
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 5, lengths=[256], H_s=8, H_r=8, H_kv=2, d=128)
    q, k = x["q_s"].copy(), x["k_s"].copy()
    k[:, 64:128] = 4.0 * q[:, 128:192]
    x["k_s"] = k
    tau = _f32(0.95)
    store, host = _compress_case(mf, x, tau, 64, "bf16")
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, 64)
    _check_compress(x, host, ref, tau, 64)


@pytest.mark.parametrize("lengths,H_s,d,B,seed", [
    ([300], 8, 64, 64, 6),                   # d = 64 with 64-token blocks
])
def test_compress_bf16_d64_b64(mf, lengths, H_s, d, B, seed):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, seed, lengths=lengths, H_s=H_s, H_r=8, H_kv=2, d=d)
    tau = _f32(0.9)
    store, host = _compress_case(mf, x, tau, B, "bf16")
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    _check_compress(x, host, ref, tau, B)


def _upload_oracle_store(mf, ref, x):
    store = mf.BlockStore.create(ref.H_s, ref.B, x["cu_seqlens"], capacity=len(ref.block_idx))
    store.upload(ref.block_ptr, ref.block_idx, ref.probs, ref.row_kept_mass)
    return store


@pytest.mark.parametrize("case", [
    dict(wl="tiny", seed=0, lengths=None, heads=None),
    dict(wl="tiny", seed=1, lengths=None, heads=None),
    dict(wl="tiny", seed=2, lengths=None, heads=None),
    dict(wl="pair_8b3b_8k", seed=0, lengths=[357], heads=(32, 24, 8, 128)),
    dict(wl="pair_8b3b_8k", seed=1, lengths=[130, 1, 64, 250], heads=(32, 24, 8, 128)),
    dict(wl="varlen_14b8b", seed=0, lengths=[333, 70], heads=(40, 32, 8, 128)),
    dict(wl="pair_8b3b_8k", seed=2, lengths=[200], heads=(16, 12, 4, 64)),
    dict(wl="pair_8b3b_8k", seed=3, lengths=[190], heads=(8, 5, 5, 128)),
    dict(wl="pair_8b3b_8k", seed=4, lengths=[170, 33], heads=(16, 48, 8, 64)),   # 48 heads: split
    dict(wl="varlen_14b8b", seed=1, lengths=[150], heads=(40, 25, 5, 128)),      # split, 1 head left
    # 32 heads: one half-block workgroup (KV groups of 4), or two 16-head splits (KV groups of 2)
    dict(wl="pair_8b3b_8k", seed=11, lengths=[260, 3, 129], heads=(32, 32, 4, 128)),
    dict(wl="varlen_14b8b", seed=12, lengths=[211], heads=(40, 32, 16, 128)),
    dict(wl="pair_8b3b_8k", seed=13, lengths=[160], heads=(48, 32, 8, 64)),
    # 33..48 sender heads: the last head chunk's hi and lo weights share one product
    dict(wl="varlen_14b8b", seed=14, lengths=[190, 40], heads=(36, 8, 8, 128)),
    dict(wl="varlen_14b8b", seed=15, lengths=[230], heads=(44, 16, 4, 64)),
])
def test_retrieve_on_oracle_store(mf, case):
    wl = synth.WORKLOADS[case["wl"]]
    kw = {}
    if case["heads"]:
        kw = dict(zip(["H_s", "H_r", "H_kv", "d"], case["heads"]))
    x = synth.make_layer_inputs(wl, case["seed"], lengths=case["lengths"], **kw)
    tau = _f32(wl.tau)
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
    say(f"case: retrieve {case} nnzb={len(ref.block_idx)}")
    store = _upload_oracle_store(mf, ref, x)
    W, V = to_dev(x["w"]), to_dev(x["v_r"], wl.dtype)
    O = mf.retrieve(store, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    ref_O = oracle.retrieve(ref, x["w"], x["v_r"], x["kv_head_map"])
    assert_out_close(O.cpu().numpy(), ref_O, "O_r")
    # a permuted kv map exercises the head ordering
    if x["H_kv"] > 1:
        kvm = x["kv_head_map"][::-1].copy()
        O2 = mf.retrieve(store, W, V, kvm)
        torch.cuda.synchronize()
        assert_out_close(O2.cpu().numpy(), oracle.retrieve(ref, x["w"], x["v_r"], kvm), "O_r (reversed kv map)")


def _random_shape(k):
    """Shape k of a seeded sweep over what the retrieve accepts: B 32 or 64, d 64 or 128, 1..64
    sender heads, 1..48 receiver heads with 1..H_r KV heads, 1..3 ragged sequences."""
    r = np.random.default_rng(np.random.SeedSequence([4242, k]))
    B = int(r.choice([32, 64]))
    d = int(r.choice([64, 128]))
    H_s = int(r.integers(1, 65))
    H_r = int(r.integers(1, 49))
    H_kv = int(r.choice([h for h in range(1, H_r + 1) if H_r % h == 0]))
    lengths = [int(n) for n in r.integers(1, 3 * B + 40, size=int(r.integers(1, 4)))]
    return B, d, H_s, H_r, H_kv, lengths


@pytest.mark.parametrize("k", range(40))
def test_retrieve_random_shapes(mf, k):
    """A seeded sweep of shapes through the head-split planner and every kernel path (whole-block
    and half-block fast paths, the general path, one or two head chunks, split receivers),
    each against the oracle's retrieve on the oracle's own store."""
    B, d, H_s, H_r, H_kv, lengths = _random_shape(k)
    wl = synth.WORKLOADS["tiny" if B == 32 else "pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 300 + k, lengths=lengths, H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
    tau = _f32(wl.tau)
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    say(f"case: random shape {k}: B={B} d={d} H_s={H_s} H_r={H_r} H_kv={H_kv} lengths={lengths} "
        f"nnzb={len(ref.block_idx)}")
    store = _upload_oracle_store(mf, ref, x)
    O = mf.retrieve(store, to_dev(x["w"]), to_dev(x["v_r"], wl.dtype), x["kv_head_map"])
    torch.cuda.synchronize()
    assert_out_close(O.cpu().numpy(), oracle.retrieve(ref, x["w"], x["v_r"], x["kv_head_map"]), "O_r")


@pytest.mark.parametrize("case", [
    # 14B-like sender fanned out to an 8B-like receiver (one 32-head part on the half-block path)
    # and two small ones
    dict(wl="varlen_14b8b", seed=2, lengths=[260, 45], H_s=40, d=128, recv=[(32, 8), (16, 2), (5, 5)]),
    # 24 heads (one part) next to 48 heads (two parts), both at 3 heads per wave
    dict(wl="pair_8b3b_8k", seed=5, lengths=[300], H_s=32, d=128, recv=[(24, 8), (48, 8)]),
    # four receivers, B = 32, ragged lengths with a one-token sequence
    dict(wl="tiny", seed=6, lengths=[90, 1, 75], H_s=16, d=64, recv=[(8, 2), (12, 4), (16, 8), (3, 1)]),
])
def test_retrieve_multi(mf, case):
    """One launch for several receivers equals one retrieve per receiver, bit for bit, and the
    oracle per receiver."""
    wl = synth.WORKLOADS[case["wl"]]
    H_s, d = case["H_s"], case["d"]
    xs = [synth.make_layer_inputs(wl, case["seed"], layer=r, lengths=case["lengths"], H_s=H_s,
                                  H_r=H_r, H_kv=H_kv, d=d)
          for r, (H_r, H_kv) in enumerate(case["recv"])]
    x = xs[0]
    tau = _f32(wl.tau)
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
    say(f"case: retrieve_multi {case} nnzb={len(ref.block_idx)}")
    store = _upload_oracle_store(mf, ref, x)
    recvs, singles = [], []
    for xr in xs:
        W = to_dev(xr["w"])
        pv = mf.v_prepare(to_dev(xr["v_r"], wl.dtype), wl.B, cu_seqlens=xr["cu_seqlens"])
        recvs.append((W, pv, xr["kv_head_map"]))
        singles.append(mf.retrieve_prepared(store, W, pv, xr["kv_head_map"]))
    outs = mf.retrieve_multi(store, recvs)
    torch.cuda.synchronize()
    for r, xr in enumerate(xs):
        assert torch.equal(outs[r], singles[r]), f"receiver {r}"
        assert_out_close(outs[r].cpu().numpy(), oracle.retrieve(ref, xr["w"], xr["v_r"], xr["kv_head_map"]),
                         f"O_r receiver {r}")
    with pytest.raises(RuntimeError):
        mf.retrieve_multi(store, recvs[:1] * 5)          # more receivers than one launch takes


@pytest.mark.parametrize("k", range(12))
def test_retrieve_multi_random(mf, k):
    """Seeded fan-outs of 1..4 receivers with random head counts and KV groupings: the planner's
    parts, packings and launch widths must leave every receiver bit-identical to its own retrieve
    and within tolerance of the oracle."""
    r = np.random.default_rng(np.random.SeedSequence([4444, k]))
    B = int(r.choice([32, 64]))
    d = int(r.choice([64, 128]))
    H_s = int(r.integers(1, 65))
    recv = []
    for _ in range(int(r.integers(1, 5))):
        H_r = int(r.integers(1, 49))
        recv.append((H_r, int(r.choice([h for h in range(1, H_r + 1) if H_r % h == 0]))))
    lengths = [int(n) for n in r.integers(1, 3 * B + 40, size=int(r.integers(1, 4)))]
    wl = synth.WORKLOADS["tiny" if B == 32 else "pair_8b3b_8k"]
    xs = [synth.make_layer_inputs(wl, 700 + k, layer=j, lengths=lengths, H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
          for j, (H_r, H_kv) in enumerate(recv)]
    x = xs[0]
    tau = _f32(wl.tau)
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    say(f"case: random fan-out {k}: B={B} d={d} H_s={H_s} receivers={recv} lengths={lengths}")
    store = _upload_oracle_store(mf, ref, x)
    recvs, singles = [], []
    for xr in xs:
        W = to_dev(xr["w"])
        pv = mf.v_prepare(to_dev(xr["v_r"], wl.dtype), B, cu_seqlens=xr["cu_seqlens"])
        recvs.append((W, pv, xr["kv_head_map"]))
        singles.append(mf.retrieve_prepared(store, W, pv, xr["kv_head_map"]))
    outs = mf.retrieve_multi(store, recvs)
    torch.cuda.synchronize()
    for j, xr in enumerate(xs):
        assert torch.equal(outs[j], singles[j]), f"receiver {j}"
        assert_out_close(outs[j].cpu().numpy(), oracle.retrieve(ref, xr["w"], xr["v_r"], xr["kv_head_map"]),
                         f"O_r receiver {j}")


@pytest.mark.parametrize("case", [
    dict(wl="tiny", seed=8, lengths=[90, 1, 75], H_s=4, d=64, dtype="f32"),
    dict(wl="pair_8b3b_8k", seed=9, lengths=[200, 70], H_s=8, d=128, dtype="bf16"),
    dict(wl="pair_8b3b_8k", seed=10, lengths=[129], H_s=16, d=64, dtype="bf16"),
])
def test_compress_prefill(mf, case):
    """The fused sender prefill fills the store like the plain compress: both stores pass the
    oracle's compress checks (their statistics use different reference maxima, so they agree up
    to rounding, not bit for bit), and the sender's attention output matches the oracle's causal
    attention of the sender heads."""
    wl = synth.WORKLOADS[case["wl"]]
    H_s, d = case["H_s"], case["d"]
    x = synth.make_layer_inputs(wl, case["seed"], lengths=case["lengths"], H_s=H_s, H_r=2, H_kv=1, d=d)
    v = synth.make_dense_inputs(wl, case["seed"], layer=1, lengths=case["lengths"], H_q=H_s, H_kv=H_s, d=d)["v"]
    tau = _f32(wl.tau)
    say(f"case: prefill {case}")
    Q, K, V = to_dev(x["q_s"], case["dtype"]), to_dev(x["k_s"], case["dtype"]), to_dev(v, case["dtype"])
    plain = mf.BlockStore.create(H_s, wl.B, x["cu_seqlens"])
    fused = mf.BlockStore.create(H_s, wl.B, x["cu_seqlens"])
    mf.compress_into(plain, Q, K, tau)
    O = mf.compress_prefill_into(fused, Q, K, V, tau)
    plain.sync()
    fused.sync()
    hp, hf = plain.to_host(), fused.to_host()
    ref_c = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
    _check_compress(x, hp, ref_c, tau, wl.B)
    _check_compress(x, hf, ref_c, tau, wl.B)
    ref = oracle.dense_causal_attention(x["q_s"].transpose(1, 0, 2), x["k_s"].transpose(1, 0, 2), v,
                                        x["cu_seqlens"], list(range(H_s)))
    assert_out_close(O.cpu().numpy(), ref, "sender O")


@pytest.mark.parametrize("k", range(8))
def test_compress_prefill_random_shapes(mf, k):
    """Seeded shapes through the fused sender prefill: its store passes the oracle's compress
    checks and its attention output matches the oracle's causal attention of the sender heads."""
    r = np.random.default_rng(np.random.SeedSequence([4747, k]))
    B = int(r.choice([32, 64]))
    d = int(r.choice([64, 128]))
    H_s = int(r.integers(1, 25))
    dtype = str(r.choice(["bf16", "f32"]))
    lengths = [int(n) for n in r.integers(1, 3 * B + 40, size=int(r.integers(1, 4)))]
    wl = synth.WORKLOADS["tiny" if dtype == "f32" else "pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 600 + k, lengths=lengths, H_s=H_s, H_r=2, H_kv=1, d=d)
    v = synth.make_dense_inputs(wl, 600 + k, layer=1, lengths=lengths, H_q=H_s, H_kv=H_s, d=d)["v"]
    tau = _f32(r.uniform(0.5, 1.0))
    say(f"case: random prefill {k}: B={B} d={d} H_s={H_s} {dtype} tau={tau} lengths={lengths}")
    Q, K, V = to_dev(x["q_s"], dtype), to_dev(x["k_s"], dtype), to_dev(v, dtype)
    fused = mf.BlockStore.create(H_s, B, x["cu_seqlens"])
    O = mf.compress_prefill_into(fused, Q, K, V, tau)
    fused.sync()
    ref_c = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    _check_compress(x, fused.to_host(), ref_c, tau, B)
    ref = oracle.dense_causal_attention(x["q_s"].transpose(1, 0, 2), x["k_s"].transpose(1, 0, 2), v,
                                        x["cu_seqlens"], list(range(H_s)))
    assert_out_close(O.cpu().numpy(), ref, "sender O")


@pytest.mark.parametrize("k", range(6))
def test_retrieve_paged_random(mf, k):
    """Seeded page sizes and page-table shuffles: a paged V pool gives the contiguous V's output
    bit for bit."""
    r = np.random.default_rng(np.random.SeedSequence([4848, k]))
    page = int(r.choice([1, 8, 16, 64, 256]))
    lengths = [int(n) for n in r.integers(1, 400, size=int(r.integers(1, 6)))]
    H_r = int(r.integers(1, 33))
    H_kv = int(r.choice([h for h in range(1, H_r + 1) if H_r % h == 0]))
    wl = synth.WORKLOADS["varlen_14b8b"]
    x = synth.make_layer_inputs(wl, 950 + k, lengths=lengths, H_s=int(r.integers(1, 41)), H_r=H_r, H_kv=H_kv,
                                d=int(r.choice([64, 128])))
    tau = _f32(wl.tau)
    say(f"case: random paged {k}: page={page} lengths={lengths} H_r={H_r} H_kv={H_kv}")
    store = mf.compress(to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16"), tau, wl.B, cu_seqlens=x["cu_seqlens"])
    W = to_dev(x["w"])
    O = mf.retrieve(store, W, to_dev(x["v_r"], "bf16"), x["kv_head_map"])
    table, n_pages = synth.make_page_table(lengths, page, seed=950 + k)
    pool = synth.page_v(x["v_r"], lengths, table, page, n_pages)
    Op = mf.retrieve(store, W, to_dev(pool, "bf16"), x["kv_head_map"],
                     page_table=torch.from_numpy(table).cuda(), page_size=page)
    torch.cuda.synchronize()
    assert torch.equal(O, Op)


def test_retrieve_paged_equals_contiguous_and_varlen_equals_per_sequence(mf):
    wl = synth.WORKLOADS["varlen_14b8b"]
    lengths = [300, 17, 129]
    x = synth.make_layer_inputs(wl, 5, lengths=lengths, H_s=16, H_r=8, H_kv=4, d=128)
    tau = _f32(wl.tau)
    say(f"case: paged/varlen lengths={lengths}")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    store = mf.compress(Q, K, tau, wl.B, cu_seqlens=x["cu_seqlens"])
    O = mf.retrieve(store, W, V, x["kv_head_map"])
    table, n_pages = synth.make_page_table(lengths, 16, seed=5)
    pool = synth.page_v(x["v_r"], lengths, table, 16, n_pages)
    Op = mf.retrieve(store, W, to_dev(pool, "bf16"), x["kv_head_map"],
                     page_table=torch.from_numpy(table).cuda(), page_size=16)
    torch.cuda.synchronize()
    assert torch.equal(O, Op)
    cu = x["cu_seqlens"]
    for s, n in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        st = mf.compress(Q[:, a:b].contiguous(), K[:, a:b].contiguous(), tau, wl.B)
        Os = mf.retrieve(st, W, V[a:b].contiguous(), x["kv_head_map"])
        torch.cuda.synchronize()
        assert torch.equal(Os, O[a:b]), f"sequence {s}"


@pytest.mark.parametrize("H_s", [32, 36, 40])
def test_batch_store_equals_per_sequence_stores(mf, H_s):
    """A batch of many sequences is large enough for the gather and the statistics to regroup
    their work orders by sequence (at least 64 L rows, 256 L pairs); every row's kept blocks,
    probabilities and kept mass, and the retrieve output, must equal those of the sequences
    compressed one at a time (row results do not depend on the order the rows run in)."""
    wl = synth.WORKLOADS["varlen_14b8b"]
    lengths = [int(n) for n in np.random.default_rng(20 + H_s).integers(900, 1500, size=40)]
    x = synth.make_layer_inputs(wl, 20 + H_s, lengths=lengths, H_s=H_s, H_r=8, H_kv=2, d=64)
    tau = np.float32(0.6).item()          # few kept blocks: the host copies stay small
    cu = x["cu_seqlens"]
    say(f"case: batch of {len(lengths)} sequences, H_s={H_s}, T={int(cu[-1])}")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    store = mf.compress(Q, K, tau, wl.B, cu_seqlens=cu)
    O = mf.retrieve(store, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    meta = store.meta_to_host()
    assert int(meta["block_ptr"][-1]) == meta["nnzb"]
    row0 = 0
    for s_, n in enumerate(lengths):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        st = mf.compress(Q[:, a:b].contiguous(), K[:, a:b].contiguous(), tau, wl.B)
        Os = mf.retrieve(st, W, V[a:b].contiguous(), x["kv_head_map"])
        torch.cuda.synchronize()
        hs = st.to_host()
        nb = (n + wl.B - 1) // wl.B
        lo, hi = int(meta["block_ptr"][row0]), int(meta["block_ptr"][row0 + nb])
        assert np.array_equal(meta["block_ptr"][row0:row0 + nb + 1] - lo, hs["block_ptr"]), f"sequence {s_}"
        blk = store.blocks_to_host(lo, hi - lo)
        assert np.array_equal(blk["block_idx"], hs["block_idx"]), f"sequence {s_}"
        assert np.array_equal(blk["probs"], hs["probs"]), f"sequence {s_}"
        assert np.array_equal(meta["row_kept_mass"][:, a:b], hs["row_kept_mass"]), f"sequence {s_}"
        assert torch.equal(Os, O[a:b]), f"sequence {s_}"
        row0 += nb


def test_end_to_end_and_determinism(mf):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 7, lengths=[420], H_s=32, H_r=24, H_kv=8, d=128)
    tau = _f32(wl.tau)
    say("case: end-to-end L=420 32->24/8")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    s1 = mf.compress(Q, K, tau, wl.B)
    O1 = mf.retrieve(s1, W, V, x["kv_head_map"])
    s2 = mf.compress(Q, K, tau, wl.B)
    O2 = mf.retrieve(s2, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    h1, h2 = s1.to_host(), s2.to_host()
    for key in ["block_ptr", "block_idx", "probs_bits", "row_kept_mass"]:
        assert np.array_equal(h1[key], h2[key]), key
    assert torch.equal(O1, O2)
    # every row's kept set against the oracle's (tie rule), then the output against the oracle run
    # on the GPU's own stored blocks, whether or not some row was a tie
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
    ex = check_selection(h1, ref, tau, wl.B)
    gs = gpu_store_for_oracle(h1, x["cu_seqlens"], wl.B, x["H_s"])
    assert_out_close(O1.cpu().numpy(), oracle.retrieve(gs, x["w"], x["v_r"], x["kv_head_map"]),
                     f"end-to-end O_r ({ex} tie rows)")


def test_compress_into_capacity(mf):
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_layer_inputs(wl, 0)
    tau = _f32(wl.tau)
    say("case: compress_into capacity")
    Q, K = to_dev(x["q_s"]), to_dev(x["k_s"])
    full = mf.BlockStore.create(wl.H_s, wl.B, x["cu_seqlens"], capacity=-1)
    mf.compress_into(full, Q, K, tau)
    n = full.sync()
    ref = mf.compress(Q, K, tau, wl.B)
    h_full, h_ref = full.to_host(), ref.to_host()
    assert n == h_ref["nnzb"]
    for key in ["block_ptr", "block_idx", "probs_bits", "row_kept_mass"]:
        assert np.array_equal(h_full[key], h_ref[key]), key
    small = mf.BlockStore.create(wl.H_s, wl.B, x["cu_seqlens"], capacity=n - 1)
    mf.compress_into(small, Q, K, tau)
    with pytest.raises(mf.MapflowError, match="CAPACITY"):
        small.sync()


@pytest.mark.parametrize("lengths,Hq,Hkv,d,dtype", [
    ([300], 24, 8, 128, "bf16"),
    ([64, 1, 190], 6, 2, 64, "bf16"),
    ([130], 4, 4, 64, "f32"),
])
def test_dense_attention(mf, lengths, Hq, Hkv, d, dtype):
    wl = synth.WORKLOADS["full_8b3b_32k"]
    x = synth.make_dense_inputs(wl, 0, layer=0, lengths=lengths, H_q=Hq, H_kv=Hkv, d=d)
    say(f"case: dense lengths={lengths} {Hq}/{Hkv} d={d} {dtype}")
    kv = [g // (Hq // Hkv) for g in range(Hq)]
    q = x["q"] if dtype == "bf16" else x["q"]
    O = mf.dense_attention(to_dev(q, dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype), kv,
                           cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"], x["cu_seqlens"], kv)
    assert_out_close(O.cpu().numpy(), ref, "dense O")


@pytest.mark.parametrize("k", range(10))
def test_dense_attention_random_shapes(mf, k):
    """Seeded dense recompute shapes: 1..32 query heads over a divisor number of KV heads, d 64 or
    128, bf16 or fp32, 1..3 ragged sequences, against the oracle's causal attention."""
    r = np.random.default_rng(np.random.SeedSequence([4545, k]))
    Hq = int(r.integers(1, 33))
    Hkv = int(r.choice([h for h in range(1, Hq + 1) if Hq % h == 0]))
    d = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    lengths = [int(n) for n in r.integers(1, 300, size=int(r.integers(1, 4)))]
    wl = synth.WORKLOADS["full_8b3b_32k"]
    x = synth.make_dense_inputs(wl, 900 + k, layer=0, lengths=lengths, H_q=Hq, H_kv=Hkv, d=d)
    say(f"case: random dense {k}: lengths={lengths} {Hq}/{Hkv} d={d} {dtype}")
    kv = [g // (Hq // Hkv) for g in range(Hq)]
    O = mf.dense_attention(to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype), kv,
                           cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    assert_out_close(O.cpu().numpy(), oracle.dense_causal_attention(x["q"], x["k"], x["v"], x["cu_seqlens"], kv),
                     "dense O")


def test_copy_probe(mf):
    src = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    mf.copy_probe(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_misaligned_inputs_are_rejected(mf):
    """Q, K and V are read with 16-byte loads: a base pointer off 16-byte alignment is an
    argument error, raised before any launch."""
    from cross_model_attention_amd import MapflowError
    H, T, d = 2, 128, 64
    flat = torch.zeros(H * T * d + 8, dtype=torch.bfloat16, device="cuda")
    good = flat[:H * T * d].view(H, T, d)
    bad = flat[1:1 + H * T * d].view(H, T, d)              # 2 bytes off
    store = mf.BlockStore.create(H, 32, [0, T])
    with pytest.raises(MapflowError):
        mf.compress_into(store, bad, good, 0.9)
    with pytest.raises(MapflowError):
        mf.compress_into(store, good, bad, 0.9)
    V = flat[1:1 + T * H * d].view(T, H, d)
    with pytest.raises(MapflowError):
        mf.v_prepare(V, 32, [0, T])
    with pytest.raises(MapflowError):
        mf.dense_attention(V, V, V, [0, 1])
    mf.compress_into(store, good, good, 0.9)               # the aligned call still works
    torch.cuda.synchronize()


def test_fill_probe_writes_every_word(mf):
    n = 3 * 262144 // 4
    dst = torch.zeros(n + 64, dtype=torch.int32, device="cuda")
    mf.fill_probe(dst[:n], 0x9E3779B9)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], torch.full((n,), 0x9E3779B9 - 2**32, dtype=torch.int32, device="cuda"))
    assert torch.count_nonzero(dst[n:]).item() == 0            # nothing past the end


def test_write_probe_pattern(mf):
    n_iter = 37
    rec = torch.arange(n_iter * 256 * 4, dtype=torch.int32, device="cuda").view(n_iter * 256, 4)
    dst = torch.zeros((n_iter * 1280, 4), dtype=torch.int32, device="cuda")
    mf.write_probe(dst, rec)
    torch.cuda.synchronize()
    u = torch.arange(5, device="cuda", dtype=torch.int32).view(1, 5, 1, 1)
    want = rec.view(n_iter, 1, 256, 4) + u
    assert torch.equal(dst.view(n_iter, 5, 256, 4), want)
    mf.write_probe(dst)
    torch.cuda.synchronize()
    it = torch.arange(n_iter, device="cuda", dtype=torch.int32).view(n_iter, 1, 1)
    base = torch.cat([it, torch.full_like(it, 7), torch.full_like(it, 8), torch.full_like(it, 9)], dim=2)
    want = base.view(n_iter, 1, 1, 4) + u
    assert torch.equal(dst.view(n_iter, 5, 256, 4), want.expand(n_iter, 5, 256, 4))


def test_read_probe_reads_without_writing(mf):
    src = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    mf.read_probe(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(sink.cpu(), torch.full((4,), 7, dtype=torch.int32))


def _rows_of(host, r):
    a, b = int(host["block_ptr"][r]), int(host["block_ptr"][r + 1])
    return host["block_idx"][a:b], host["probs_bits"][a:b]


@pytest.mark.parametrize("k", range(8))
def test_range_store_random(mf, k):
    """Seeded row ranges (a random first row per sequence, some past the last row): the range
    store's rows equal the full store's bit for bit, it keeps nothing elsewhere, and its retrieve
    writes exactly its rows, equal to the full retrieve's."""
    r = np.random.default_rng(np.random.SeedSequence([4646, k]))
    B = int(r.choice([32, 64]))
    H_s = int(r.integers(1, 41))
    lengths = [int(n) for n in r.integers(1, 6 * B, size=int(r.integers(1, 5)))]
    nbs = [(n + B - 1) // B for n in lengths]
    row_begin = [int(r.integers(0, nb + 1)) for nb in nbs]
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 800 + k, lengths=lengths, H_s=H_s, H_r=6, H_kv=2, d=64)
    tau = _f32(wl.tau)
    say(f"case: random range store {k}: B={B} H_s={H_s} lengths={lengths} row_begin={row_begin}")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    full = mf.BlockStore.create(H_s, B, x["cu_seqlens"])
    part = mf.BlockStore.create(H_s, B, x["cu_seqlens"], row_begin=row_begin)
    assert part.raw.n_order == sum(nb - rb for nb, rb in zip(nbs, row_begin))
    mf.compress_into(full, Q, K, tau)
    mf.compress_into(part, Q, K, tau)
    full.sync()
    part.sync()
    hf, hp = full.to_host(), part.to_host()
    cu = x["cu_seqlens"]
    active_tok = np.zeros(int(cu[-1]), dtype=bool)
    row = 0
    for s_, n in enumerate(lengths):
        for I in range(nbs[s_]):
            if I >= row_begin[s_]:
                for a_, b_ in zip(_rows_of(hf, row), _rows_of(hp, row)):
                    assert np.array_equal(a_, b_), f"row {row}"
                active_tok[int(cu[s_]) + I * B: int(cu[s_]) + min(n, (I + 1) * B)] = True
            else:
                assert len(_rows_of(hp, row)[0]) == 0, f"row {row} outside the range kept blocks"
            row += 1
    assert np.array_equal(hf["row_kept_mass"][:, active_tok], hp["row_kept_mass"][:, active_tok])
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    O_full = mf.retrieve(full, W, V, x["kv_head_map"])
    O_part = torch.full_like(O_full, float("nan"))
    mf.retrieve(part, W, V, x["kv_head_map"], out=O_part)
    torch.cuda.synchronize()
    act = torch.from_numpy(active_tok).cuda()
    assert torch.equal(O_part[act], O_full[act])
    assert torch.isnan(O_part[~act]).all()


def test_chunked_prefill_rows_equal_the_full_store(mf):
    """A row-range store compresses exactly the rows of the full store it covers (bit for bit),
    keeps nothing elsewhere, and its retrieve and fused prefill touch only its rows (the fused
    prefill's range rows equal those of a full fused prefill, bit for bit)."""
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    lengths = [300, 129, 64]
    x = synth.make_layer_inputs(wl, 11, lengths=lengths, H_s=8, H_r=12, H_kv=4, d=128)
    v_s = synth.make_dense_inputs(wl, 11, layer=1, lengths=lengths, H_q=8, H_kv=8, d=128)["v"]
    tau = _f32(wl.tau)
    row_begin = [2, 0, 1]                               # block rows: 5, 3, 1 (the last sequence: none)
    say(f"case: chunked prefill lengths={lengths} row_begin={row_begin}")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    full = mf.BlockStore.create(8, wl.B, x["cu_seqlens"])
    part = mf.BlockStore.create(8, wl.B, x["cu_seqlens"], row_begin=row_begin)
    assert part.raw.n_order == 3 + 3 + 0 and full.raw.n_order == full.raw.n_brow == 9
    mf.compress_into(full, Q, K, tau)
    mf.compress_into(part, Q, K, tau)
    full.sync()
    part.sync()
    hf, hp = full.to_host(), part.to_host()
    cu = x["cu_seqlens"]
    active_tok = np.zeros(int(cu[-1]), dtype=bool)
    r = 0
    for s, n in enumerate(lengths):
        for I in range((n + wl.B - 1) // wl.B):
            if I >= row_begin[s]:
                for a_, b_ in zip(_rows_of(hf, r), _rows_of(hp, r)):
                    assert np.array_equal(a_, b_), f"row {r}"
                active_tok[int(cu[s]) + I * wl.B: int(cu[s]) + min(n, (I + 1) * wl.B)] = True
            else:
                assert len(_rows_of(hp, r)[0]) == 0, f"row {r} outside the range kept blocks"
            r += 1
    assert np.array_equal(hf["row_kept_mass"][:, active_tok], hp["row_kept_mass"][:, active_tok])
    # the range store's rows against the oracle: kept sets (tie rule), every stored value against
    # the exact map, kept mass the sum of the stored values
    ref = oracle.compress(x["q_s"], x["k_s"], cu, tau, wl.B, keep_exact=True)
    r = 0
    for s_, n in enumerate(lengths):
        for I in range((n + wl.B - 1) // wl.B):
            if I >= row_begin[s_]:
                idx, bits = _rows_of(hp, r)
                ok, why = sets_agree(idx.tolist(), ref.rows[r], tau)
                assert ok, f"range row {r}: {why}"
                lo = int(hp["block_ptr"][r])
                for t, J in enumerate(idx.tolist()):
                    if J in ref.rows[r]["exact"]:
                        A = ref.rows[r]["exact"][J]
                        err = np.abs(hp["probs"][lo + t] - A)
                        assert np.all(err <= ulp_bf16(A) + 1e-6), f"range row {r} block {J}"
                rows_b, tok0 = ref.rows[r]["rows"], ref.rows[r]["tok0"]
                want = hp["probs"][lo:lo + len(idx), :, :rows_b, :].sum(axis=(0, 3))
                assert np.allclose(hp["row_kept_mass"][:, tok0:tok0 + rows_b], want, rtol=1e-6, atol=1e-7)
            r += 1
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    O_full = mf.retrieve(full, W, V, x["kv_head_map"])
    O_part = torch.full_like(O_full, float("nan"))
    mf.retrieve(part, W, V, x["kv_head_map"], out=O_part)
    torch.cuda.synchronize()
    act = torch.from_numpy(active_tok).cuda()
    assert torch.equal(O_part[act], O_full[act])
    assert torch.isnan(O_part[~act]).all()
    # the range retrieve's rows against the oracle run on the range store's own blocks
    gp = gpu_store_for_oracle(hp, cu, wl.B, 8)
    got, want = [], []
    for b, (s_, I) in enumerate(brow_table(cu, wl.B)):
        if I < row_begin[s_]:
            continue
        lo, hi = int(hp["block_ptr"][b]), int(hp["block_ptr"][b + 1])
        n = int(cu[s_ + 1] - cu[s_])
        rows_b, tok0 = min(n, (I + 1) * wl.B) - I * wl.B, int(cu[s_]) + I * wl.B
        blocks = {int(gp.block_idx[t]): gp.probs[t] for t in range(lo, hi)}
        want.append(oracle.retrieve_block_row(blocks, wl.B, rows_b, tok0, s_, int(cu[s_]), n, x["w"], x["v_r"],
                                              x["kv_head_map"]))
        got.append(O_part[tok0:tok0 + rows_b].cpu().numpy())
    assert_out_close(np.concatenate(got), np.concatenate(want), "O_r (range store)")
    # the fused prefill on the range store: same store, attention rows of the range only
    pre = mf.BlockStore.create(8, wl.B, x["cu_seqlens"], row_begin=row_begin)
    Vs = to_dev(v_s, "bf16")
    O_pre = torch.full((int(cu[-1]), 8, 128), float("nan"), device="cuda")
    mf.compress_prefill_into(pre, Q, K, Vs, tau, out=O_pre)
    pre.sync()
    pre_full = mf.BlockStore.create(8, wl.B, x["cu_seqlens"])
    O_pre_full = mf.compress_prefill_into(pre_full, Q, K, Vs, tau)
    pre_full.sync()
    torch.cuda.synchronize()
    hq, hqf = pre.to_host(), pre_full.to_host()
    assert np.array_equal(hq["block_ptr"], hp["block_ptr"])
    r = 0
    for s, n in enumerate(lengths):
        for I in range((n + wl.B - 1) // wl.B):
            if I >= row_begin[s]:
                for a_, b_ in zip(_rows_of(hqf, r), _rows_of(hq, r)):
                    assert np.array_equal(a_, b_), f"prefill row {r}"
            r += 1
    assert np.array_equal(hqf["row_kept_mass"][:, active_tok], hq["row_kept_mass"][:, active_tok])
    assert torch.equal(O_pre[act], O_pre_full[act]) and torch.isnan(O_pre[~act]).all()


@pytest.mark.parametrize("k", range(4))
def test_prefix_cache_random_requests(mf, k):
    """Seeded conversation trees through a cache small enough to evict: each request continues an
    earlier one (all of it, or up to a random point) with new tokens.  Its output, assembled from
    the looked-up prefix and a row-range store of the rest, equals compressing it whole, bit for
    bit; requests that extend a cached one find it; the cache's bytes stay within its budget."""
    r = np.random.default_rng(np.random.SeedSequence([5252, k]))
    B, H_s, H_r, H_kv, d = 64, 8, 6, 2, 64
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    tau = _f32(wl.tau)
    w = synth.make_layer_inputs(wl, 1100 + k, lengths=[B], H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
    W, kv = to_dev(w["w"]), w["kv_head_map"]
    budget = 3 << 20
    cache = mf.PrefixCache(budget)
    reqs = []                                        # (tokens, q_s, k_s, v_r) of earlier requests
    hits = 0
    for q in range(12):
        if reqs and r.random() < 0.8:
            ptok, pq, pk, pv = reqs[int(r.integers(0, len(reqs)))]
            p = len(ptok) if r.random() < 0.5 else int(r.integers(0, len(ptok) + 1))
        else:
            ptok, pq, pk, pv, p = np.zeros(0, np.int32), None, None, None, 0
        n = min(p + int(r.integers(1, 4 * B)), 12 * B)
        fresh = synth.make_layer_inputs(wl, 2000 + 100 * k + q, lengths=[n], H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
        tail = r.integers(0, 50000, size=n - p).astype(np.int32)
        if p < len(ptok) and n > p and tail[0] == ptok[p]:
            tail[0] ^= 1
        tok = np.concatenate([ptok[:p], tail])
        qs = fresh["q_s"] if p == 0 else np.concatenate([pq[:, :p], fresh["q_s"][:, p:]], axis=1)
        ks = fresh["k_s"] if p == 0 else np.concatenate([pk[:, :p], fresh["k_s"][:, p:]], axis=1)
        vs = fresh["v_r"] if p == 0 else np.concatenate([pv[:p], fresh["v_r"][p:]], axis=0)
        reqs.append((tok, qs, ks, vs))
        Q, K, V = to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16")
        rows, view = cache.lookup(0, tok, B)
        say(f"case: random cache {k} request {q}: continues {p} tokens, length {n}, cached rows {rows}")
        assert rows <= n // B
        hits += rows > 0
        part = mf.BlockStore.create(H_s, B, [0, n], row_begin=[rows])
        mf.compress_into(part, Q, K, tau)
        part.sync()
        O = torch.full((n, H_r, d), float("nan"), device="cuda")
        if rows:
            mf.retrieve(view, W, V[: rows * B].contiguous(), kv, out=O[: rows * B])
        mf.retrieve(part, W, V, kv, out=O)
        whole = mf.BlockStore.create(H_s, B, [0, n])
        mf.compress_into(whole, Q, K, tau)
        O_whole = mf.retrieve(whole, W, V, kv)
        torch.cuda.synchronize()
        assert torch.equal(O, O_whole), f"request {q}"
        if n // B > 0:
            try:
                cache.insert(0, tok, ([view] if rows else []) + [part], n // B)
            except mf.MapflowError as e:
                assert "CAPACITY" in str(e), str(e)
        assert cache.info()[1] <= budget
        del view
    say(f"  requests served from the cache: {hits}")
    assert hits > 0
    cache.close()


def test_prefix_cache_reuses_a_previous_request(mf):
    """Request 2 extends request 1: its cached prefix plus a row-range store of the new rows give
    the same retrieve output as compressing request 2 whole; inserting the combined prefix gives
    the rows of the whole compression, bit for bit."""
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    B = wl.B
    n1, n2 = 5 * B + 10, 9 * B + 3
    x = synth.make_layer_inputs(wl, 12, lengths=[n2], H_s=8, H_r=12, H_kv=4, d=128)
    tokens = np.random.default_rng(12).integers(0, 50000, size=n2, dtype=np.int32)
    tau = _f32(wl.tau)
    say(f"case: prefix cache n1={n1} n2={n2}")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    cache = mf.PrefixCache(1 << 30)
    # request 1: compress it whole, cache its complete rows
    s1 = mf.BlockStore.create(8, B, [0, n1])
    mf.compress_into(s1, Q[:, :n1].contiguous(), K[:, :n1].contiguous(), tau)
    s1.sync()
    cache.insert(3, tokens[:n1], [s1], n1 // B)
    assert cache.info()[0] == 1
    assert cache.lookup(3, tokens[:n1], B)[0] == 5
    assert cache.lookup(4, tokens[:n1], B)[0] == 0               # other layer
    changed = tokens.copy()
    changed[2 * B + 1] += 1
    assert cache.lookup(3, changed, B)[0] == 0                   # the cached prefix no longer matches
    # request 2: cached rows 0..4, new rows 5..9
    rows, view = cache.lookup(3, tokens, B)
    assert rows == 5 and view.raw.T == 5 * B
    new = mf.BlockStore.create(8, B, [0, n2], row_begin=[rows])
    mf.compress_into(new, Q, K, tau)
    new.sync()
    O = torch.empty((n2, 12, 128), device="cuda")
    mf.retrieve(view, W, V[: rows * B].contiguous(), x["kv_head_map"], out=O[: rows * B])
    mf.retrieve(new, W, V, x["kv_head_map"], out=O)
    whole = mf.BlockStore.create(8, B, [0, n2])
    mf.compress_into(whole, Q, K, tau)
    whole.sync()
    O_whole = mf.retrieve(whole, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    assert torch.equal(O, O_whole)
    # the cached-prefix rows and the range store's rows, each retrieved by the oracle from the
    # GPU's own blocks of the store that served them
    hv0, hn = view.to_host(), new.to_host()
    cu2 = [0, n2]
    want = np.zeros((n2, 12, 128))
    for I in range((n2 + B - 1) // B):
        src, b = (hv0, I) if I < rows else (hn, I)
        lo, hi = int(src["block_ptr"][b]), int(src["block_ptr"][b + 1])
        blocks = {int(src["block_idx"][t]): src["probs"][t] for t in range(lo, hi)}
        rows_b = min(n2, (I + 1) * B) - I * B
        want[I * B:I * B + rows_b] = oracle.retrieve_block_row(blocks, B, rows_b, I * B, 0, 0, n2, x["w"],
                                                               x["v_r"], x["kv_head_map"])
    assert_out_close(O.cpu().numpy(), want, "O_r (cached prefix + range store)")
    ref_c = oracle.compress(x["q_s"], x["k_s"], np.array(cu2), tau, B, keep_exact=True)
    for I in range(rows):                                  # the cached rows against the exact map
        lo, hi = int(hv0["block_ptr"][I]), int(hv0["block_ptr"][I + 1])
        ok, why = sets_agree(hv0["block_idx"][lo:hi].tolist(), ref_c.rows[I], tau)
        assert ok, f"cached row {I}: {why}"
        for t in range(lo, hi):
            A = ref_c.rows[I]["exact"].get(int(hv0["block_idx"][t]))
            if A is not None:
                assert np.all(np.abs(hv0["probs"][t] - A) <= ulp_bf16(A) + 1e-6), f"cached row {I}"
    # cache request 2's complete rows from the view and the new rows
    cache.insert(3, tokens, [view, new], n2 // B)
    rows2, view2 = cache.lookup(3, tokens, B)
    assert rows2 == 9 and cache.info()[0] == 2
    hv, hw = view2.to_host(), whole.to_host()
    nb = int(hv["block_ptr"][rows2])
    assert np.array_equal(hv["block_ptr"], hw["block_ptr"][: rows2 + 1])
    assert np.array_equal(hv["block_idx"], hw["block_idx"][:nb])
    assert np.array_equal(hv["probs_bits"], hw["probs_bits"][:nb])
    assert np.array_equal(hv["row_kept_mass"], hw["row_kept_mass"][:, : rows2 * B])
    # the oracle agrees with the cached rows
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
    assert np.array_equal(hv["block_idx"], ref.block_idx[: len(hv["block_idx"])])
    # a small budget evicts the least recently used entry
    small = mf.PrefixCache(int(cache.info()[1] * 0.8))
    small.insert(3, tokens[:n1], [s1], 5)
    small.insert(3, tokens, [view, new], 9)
    assert small.info()[0] == 1 and small.lookup(3, tokens[:n1], B)[0] == 0
    # a view belongs to the cache: the library refuses to free it
    from cross_model_attention_amd import _lib
    assert _lib.load().mf_bsr_free(None, ctypes.byref(view2.raw)) == _lib.MF_ERR_INVALID
    cache.close()
    small.close()


@pytest.mark.parametrize("case", [
    dict(wl="tiny", seed=13, lengths=[150, 1, 90], H_s=4, d=64, dtype="f32", sel=True, norm=False),
    dict(wl="pair_8b3b_8k", seed=14, lengths=[260, 70], H_s=8, d=128, dtype="bf16", sel=True, norm=False),
    dict(wl="pair_8b3b_8k", seed=15, lengths=[260, 70], H_s=8, d=128, dtype="bf16", sel=False, norm=True),
    dict(wl="pair_8b3b_8k", seed=16, lengths=[200], H_s=16, d=64, dtype="bf16", sel=True, norm=True),
])
def test_compress_variants(mf, case):
    """Per-head selection and per-head normalisation against the oracle's variants: the same kept
    sets (the union of the heads' own sets), zeros where a head did not select a block, stored
    values within one bf16 ulp of the oracle's, kept mass the sum of the stored values; then the
    unchanged retrieve against the oracle's retrieve of its own variant store."""
    wl = synth.WORKLOADS[case["wl"]]
    x = synth.make_layer_inputs(wl, case["seed"], lengths=case["lengths"], H_s=case["H_s"], H_r=6, H_kv=2,
                                d=case["d"])
    tau = _f32(wl.tau if case["wl"] != "tiny" else 0.7)
    say(f"case: compress variant {case}")
    Q, K = to_dev(x["q_s"], case["dtype"]), to_dev(x["k_s"], case["dtype"])
    store = mf.BlockStore.create(case["H_s"], wl.B, x["cu_seqlens"])
    mf.compress_into(store, Q, K, tau, per_head_select=case["sel"], per_head_norm=case["norm"])
    store.sync()
    host = store.to_host()
    ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B, keep_exact=True,
                          per_head_select=case["sel"], per_head_norm=case["norm"])
    assert np.array_equal(host["block_ptr"], ref.block_ptr)
    assert np.array_equal(host["block_idx"], ref.block_idx)
    # stored values against the exact (unrounded) map of the variant, zeros where a head did not
    # select the block
    err = np.abs(host["probs"] - ref.exact)
    assert np.all(err <= ulp_bf16(ref.exact) + 1e-6), f"max excess {(err - ulp_bf16(ref.exact)).max():.3e}"
    cu, B = x["cu_seqlens"], wl.B
    for b, (s, I) in enumerate(brow_table(cu, B)):
        n = int(cu[s + 1] - cu[s])
        tok0, rows_b = int(cu[s]) + I * B, min(n, I * B + B) - I * B
        lo, hi = host["block_ptr"][b], host["block_ptr"][b + 1]
        want = host["probs"][lo:hi, :, :rows_b, :].sum(axis=(0, 3))
        assert np.allclose(host["row_kept_mass"][:, tok0:tok0 + rows_b], want, rtol=1e-6, atol=1e-7)
    W, V = to_dev(x["w"]), to_dev(x["v_r"], case["dtype"])
    O = mf.retrieve(store, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    assert_out_close(O.cpu().numpy(), oracle.retrieve(ref, x["w"], x["v_r"], x["kv_head_map"]), "O_r (variant)")


@pytest.mark.parametrize("k", range(8))
def test_retrieve_layers_random(mf, k):
    """Seeded cross-layer mixes: 1..4 sender layers of 1..64 heads each, random receiver shapes,
    against the oracle's cross-layer retrieve on the same stores."""
    r = np.random.default_rng(np.random.SeedSequence([5050, k]))
    B = int(r.choice([32, 64]))
    d = int(r.choice([64, 128]))
    H_r = int(r.integers(1, 49))
    H_kv = int(r.choice([h for h in range(1, H_r + 1) if H_r % h == 0]))
    heads = [int(h) for h in r.integers(1, 65, size=int(r.integers(1, 5)))]
    lengths = [int(n) for n in r.integers(1, 3 * B + 40, size=int(r.integers(1, 4)))]
    wl = synth.WORKLOADS["tiny" if B == 32 else "pair_8b3b_8k"]
    tau = _f32(wl.tau)
    say(f"case: random cross-layer {k}: B={B} d={d} H_r={H_r} H_kv={H_kv} heads={heads} lengths={lengths}")
    refs, stores, Ws, Wn = [], [], [], []
    for l, H_s in enumerate(heads):
        x = synth.make_layer_inputs(wl, 1000 + k, layer=l, lengths=lengths, H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
        ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, B)
        refs.append(ref)
        stores.append(_upload_oracle_store(mf, ref, x))
        Wn.append(x["w"])
        Ws.append(to_dev(x["w"]))
    v, kv = x["v_r"], x["kv_head_map"]
    pv = mf.v_prepare(to_dev(v, wl.dtype), B, cu_seqlens=x["cu_seqlens"])
    O = mf.retrieve_layers(stores, Ws, pv, kv)
    torch.cuda.synchronize()
    assert_out_close(O.cpu().numpy(), oracle.retrieve_layers(refs, Wn, v, kv), "O_r (cross-layer)")


@pytest.mark.parametrize("case", [
    dict(wl="pair_8b3b_8k", seed=17, lengths=[230, 40], heads=[8, 16], H_r=12, H_kv=4, d=128),
    dict(wl="tiny", seed=18, lengths=[120, 1, 60], heads=[4, 4, 2], H_r=5, H_kv=5, d=64),
])
def test_retrieve_layers(mf, case):
    """One receiver layer from several sender layers' stores against the oracle's cross-layer
    retrieve (mix over the union of the layers' blocks, then renormalise)."""
    wl = synth.WORKLOADS[case["wl"]]
    tau = _f32(wl.tau if case["wl"] != "tiny" else 0.6)
    say(f"case: retrieve_layers {case}")
    refs, stores, Ws, Wn = [], [], [], []
    for l, H_s in enumerate(case["heads"]):
        x = synth.make_layer_inputs(wl, case["seed"], layer=l, lengths=case["lengths"], H_s=H_s, H_r=case["H_r"],
                                    H_kv=case["H_kv"], d=case["d"])
        ref = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], tau, wl.B)
        refs.append(ref)
        stores.append(_upload_oracle_store(mf, ref, x))
        Wn.append(x["w"])
        Ws.append(to_dev(x["w"]))
    v, kv = x["v_r"], x["kv_head_map"]
    pv = mf.v_prepare(to_dev(v, wl.dtype), wl.B, cu_seqlens=x["cu_seqlens"])
    O = mf.retrieve_layers(stores, Ws, pv, kv)
    torch.cuda.synchronize()
    assert_out_close(O.cpu().numpy(), oracle.retrieve_layers(refs, Wn, v, kv), "O_r (cross-layer)")
    # one layer is the plain retrieve
    O1 = mf.retrieve_layers(stores[:1], Ws[:1], pv, kv)
    torch.cuda.synchronize()
    assert torch.equal(O1, mf.retrieve_prepared(stores[0], Ws[0], pv, kv))
