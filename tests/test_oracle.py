"""Pins for the fp64 oracle, independent of the oracle's own code (CPU only, no GPU).

Each pin is one of: a library routine (torch / scipy in fp64), brute force on tiny inputs written
with scalar loops, a closed form, or an invariant the mathematics fixes.  The mutation tests at
the bottom plant plausible mistakes in the oracle and check that some pin catches each one.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle import mapflow_oracle as mo


def _rand_qk(rng, H, n, d, boost=2.0):
    q = rng.standard_normal((H, n, d))
    k = rng.standard_normal((H, n, d))
    u = rng.standard_normal((H, 1, d))
    return q + boost * u, k + boost * u


# ------------------------------------------------------------------------------------ bf16 rounding
def test_bf16_round_closed_forms():
    one = 1.0
    cases = {
        one: one,
        one + 2.0 ** -8: one,                          # tie -> even (mantissa 0)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,          # tie -> even (mantissa 2)
        one + 2.0 ** -8 + 2.0 ** -30: one + 2.0 ** -7,  # just above the tie
        one - 2.0 ** -10: one,                          # rounds up across the binade edge
        0.0: 0.0,
        -0.75: -0.75,
        1.5 * 2.0 ** -133: 2.0 * 2.0 ** -133,          # subnormal tie -> even
        2.5 * 2.0 ** -133: 2.0 * 2.0 ** -133,
        1e-50: 0.0,
    }
    for x, want in cases.items():
        assert mo.bf16_round(np.array([x]))[0] == want, x


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000), rng.random(20000) * 1e-3,
                        np.exp(rng.uniform(-80, 0, 20000))]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = mo.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------ scores, softmax, lse
def test_attention_rows_vs_library_routines():
    rng = np.random.default_rng(2)
    n, d = 70, 16
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    A, lse = mo.attention_rows(q, k, 0, n)
    s = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(d)
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    ref = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=1).numpy()
    assert np.allclose(A, ref, rtol=0, atol=1e-13)
    ref_lse = np.array([scipy.special.logsumexp(s.numpy()[i, : i + 1]) for i in range(n)])
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-12)
    # a row slice equals the same rows of the full map
    A2, lse2 = mo.attention_rows(q, k, 20, 45)
    assert np.allclose(A2, A[20:45, :45], atol=1e-15) and np.allclose(lse2, lse[20:45], atol=1e-13)


def test_attention_rows_scalar_brute_force():
    rng = np.random.default_rng(3)
    n, d = 9, 5
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    A, _ = mo.attention_rows(q, k, 0, n)
    for i in range(n):
        sc = [sum(q[i, t] * k[j, t] for t in range(d)) / math.sqrt(d) for j in range(i + 1)]
        z = sum(math.exp(x) for x in sc)
        for j in range(n):
            want = math.exp(sc[j]) / z if j <= i else 0.0
            assert abs(A[i, j] - want) < 1e-14


# --------------------------------------------------------------------- block masses and selection
def _brute_block_masses(Q, K, B, I, seq_len):
    """Scalar-loop triple sums, independent of the oracle's vectorised code."""
    H, _, d = Q.shape
    r0, r1 = I * B, min(seq_len, (I + 1) * B)
    M = [0.0] * (I + 1)
    for h in range(H):
        for i in range(r0, r1):
            sc = [float(np.dot(Q[h, i], K[h, j])) / math.sqrt(d) for j in range(i + 1)]
            mx = max(sc)
            z = sum(math.exp(x - mx) for x in sc)
            for j in range(i + 1):
                M[j // B] += math.exp(sc[j] - mx) / z
    return np.array(M)


def test_block_masses_brute_force_and_conservation():
    rng = np.random.default_rng(4)
    H, n, d, B = 2, 45, 6, 8                            # ragged last block (45 = 5*8 + 5)
    Q, K = _rand_qk(rng, H, n, d)
    for I in [0, 1, 3, 5]:
        r = mo.block_row_compress(Q, K, 0, n, I, B, tau=0.5)
        assert np.allclose(r["M"], _brute_block_masses(Q, K, B, I, n), rtol=1e-12, atol=1e-14)
        assert abs(r["M"].sum() - r["T_I"]) < 1e-12 * r["T_I"]
        assert r["T_I"] == H * (min(n, (I + 1) * B) - I * B)


def _brute_select(masses, I, T_I, tau):
    """Exhaustive search: smallest superset of the forced blocks reaching tau * T_I; among the
    smallest, the one of largest mass."""
    forced = {0, I}
    free = [J for J in range(I + 1) if J not in forced]
    best = None
    for r in range(len(free) + 1):
        for combo in itertools.combinations(free, r):
            S = forced | set(combo)
            m = sum(masses[J] for J in S)
            if m >= tau * T_I and (best is None or m > best[1]):
                best = (S, m)
        if best is not None:
            return sorted(best[0])
    return sorted(forced | set(free))


def test_selection_brute_force_small_rows():
    rng = np.random.default_rng(5)
    for trial in range(300):
        I = int(rng.integers(0, 8))
        masses = rng.random(I + 1) ** 3
        T_I = float(masses.sum())
        tau = float(rng.uniform(0.05, 0.999))
        got = mo.select_blocks(masses, I, T_I, tau)["kept"]
        assert got == _brute_select(masses, I, T_I, tau), (trial, I, tau)


def test_selection_invariants():
    rng = np.random.default_rng(6)
    for _ in range(100):
        I = int(rng.integers(0, 40))
        masses = rng.random(I + 1) ** 4
        T_I = float(masses.sum())
        taus = sorted(rng.uniform(0.01, 0.99, 5))
        sets = [set(mo.select_blocks(masses, I, T_I, t)["kept"]) for t in taus]
        for S in sets:
            assert {0, I} <= S                                           # forced blocks
        for a, b in zip(sets, sets[1:]):
            assert a <= b                                                # nested in tau
        assert mo.select_blocks(masses, I, T_I, 1.0)["kept"] == list(range(I + 1))
        assert mo.select_blocks(masses, I, T_I, 1e-12)["kept"] == sorted({0, I})


def test_selection_ties_prefer_lower_column():
    masses = np.array([0.1, 0.3, 0.3, 0.3, 0.1])
    got = mo.select_blocks(masses, 4, 1.1, tau=(0.2 + 0.3) / 1.1)["kept"]
    assert got == [0, 1, 4]
    got = mo.select_blocks(masses, 4, 1.1, tau=(0.2 + 0.6) / 1.1)["kept"]
    assert got == [0, 1, 2, 4]


def test_hand_derived_example():
    """Closed form: with d=1, q_i = 1 and k_j = ln w_j, the map is A[i, j] = w_j / sum_{j'<=i} w_j'.

    Two heads with w = (1..6) and w = (6..1), B = 2; block row 2 holds rows 4 and 5.  All values
    below are exact rationals derived by hand from that formula.
    """
    n, B = 6, 2
    w = [[Fraction(x) for x in range(1, 7)], [Fraction(x) for x in range(6, 0, -1)]]
    Q = np.ones((2, n, 1))
    K = np.array([[[math.log(float(x))] for x in wh] for wh in w])

    def A(h, i, j):
        return w[h][j] / sum(w[h][: i + 1]) if j <= i else Fraction(0)

    M_exact = [sum(A(h, i, j) for h in range(2) for i in (4, 5) for j in (2 * J, 2 * J + 1))
               for J in range(3)]
    r = mo.block_row_compress(Q, K, 0, n, 2, B, tau=0.5)
    assert np.allclose(r["M"], [float(m) for m in M_exact], rtol=0, atol=1e-14)
    forced = M_exact[0] + M_exact[2]
    total = Fraction(4)
    # forced blocks already reach tau = forced / total - 1e-9; one more block needed just above
    tau_lo = float(forced / total) - 1e-9
    tau_hi = float(forced / total) + 1e-9
    assert mo.block_row_compress(Q, K, 0, n, 2, B, tau_lo)["kept"] == [0, 2]
    assert mo.block_row_compress(Q, K, 0, n, 2, B, tau_hi)["kept"] == [0, 1, 2]
    # retrieve with H_r = 1, W = (1/4, 3/4), V[j] = j, tau = 1 (every block kept), unrounded
    bsr = mo.compress(Q, K, np.array([0, n]), tau=1.0, B=B, keep_exact=True)
    Wm = [[Fraction(1, 4), Fraction(3, 4)]]
    V = np.arange(n, dtype=float).reshape(n, 1, 1)
    O = mo.retrieve(bsr, np.array([[0.25, 0.75]]), V, [0], unrounded=True)
    for i in range(n):
        mix = [sum(Wm[0][h] * A(h, i, j) for h in range(2)) for j in range(n)]
        want = sum(mix[j] * j for j in range(n)) / sum(mix)
        assert abs(O[i, 0, 0] - float(want)) < 1e-13


# ----------------------------------------------------------------------- probs and kept row mass
def test_probs_are_rounded_map_and_row_mass_is_their_sum():
    rng = np.random.default_rng(7)
    H, n, d, B = 3, 77, 8, 16
    Q, K = _rand_qk(rng, H, n, d)
    bsr = mo.compress(Q, K, np.array([0, n]), tau=0.8, B=B, keep_exact=True)
    # stored values are bf16 numbers (fp32 -> bf16 round trip through torch is the identity)
    p32 = torch.from_numpy(bsr.probs.astype(np.float32))
    assert np.array_equal(p32.to(torch.bfloat16).to(torch.float64).numpy(), bsr.probs)
    # and within half a bf16 ulp of the exact map
    ex = bsr.exact
    half_ulp = np.where(ex > 0, np.ldexp(1.0, np.frexp(ex)[1] - 9), 0.0)
    assert np.all(np.abs(bsr.probs - ex) <= half_ulp + 1e-300)
    # row_kept_mass is the explicit sum of the stored values of each row's kept blocks
    for b in range(len(bsr.brow_I)):
        I = int(bsr.brow_I[b])
        rows = min(n, (I + 1) * B) - I * B
        for h in range(H):
            for r_ in range(rows):
                want = sum(float(bsr.probs[t, h, r_, c])
                           for t in range(bsr.block_ptr[b], bsr.block_ptr[b + 1]) for c in range(B))
                assert abs(bsr.row_kept_mass[h, I * B + r_] - want) < 1e-14
    # at tau = 1 every row keeps all its mass up to bf16 rounding
    full = mo.compress(Q, K, np.array([0, n]), tau=1.0, B=B)
    assert np.all(np.abs(full.row_kept_mass - 1.0) <= 2.0 ** -8)


# ------------------------------------------------------------------------------- retrieve pins
def test_identity_map_at_full_density_is_dense_causal_attention():
    """I2: tau = 1, H_r = H_s, W = I, kv map = identity, exact map -> SDPA (is_causal)."""
    rng = np.random.default_rng(8)
    H, n, d, B = 3, 50, 8, 16
    Q, K = _rand_qk(rng, H, n, d)
    V = rng.standard_normal((n, H, d))
    bsr = mo.compress(Q, K, np.array([0, n]), tau=1.0, B=B, keep_exact=True)
    O = mo.retrieve(bsr, np.eye(H), V, list(range(H)), unrounded=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V.transpose(1, 0, 2).copy()),
        is_causal=True).numpy().transpose(1, 0, 2)
    assert np.allclose(O, ref, rtol=0, atol=1e-12)


def test_dirichlet_rows_sum_to_one_without_renormalisation():
    """I3: at tau = 1 on the exact map every mixed row sums to sum_h W[g, h] = 1."""
    rng = np.random.default_rng(9)
    H, n, d, B = 4, 40, 8, 8
    Q, K = _rand_qk(rng, H, n, d)
    W = rng.dirichlet(np.full(H, 0.5), size=3)
    bsr = mo.compress(Q, K, np.array([0, n]), tau=1.0, B=B, keep_exact=True)
    for b in range(len(bsr.brow_I)):
        I = int(bsr.brow_I[b])
        rows = min(n, (I + 1) * B) - I * B
        blocks = {int(bsr.block_idx[t]): bsr.exact[t] for t in range(bsr.block_ptr[b], bsr.block_ptr[b + 1])}
        P, _ = mo.gather_row_probs(blocks, B, rows, 0, n)
        Ahat = mo.mix_heads(P, W)
        assert np.allclose(Ahat.sum(axis=2), 1.0, atol=1e-13)
        Abar, den = mo.renormalise(Ahat)
        assert np.allclose(Abar.sum(axis=2), 1.0, atol=1e-14)
    # renormalised rows sum to 1 for any W with a non-zero denominator, at any tau
    W2 = rng.standard_normal((3, H)) + 2.0
    part = mo.compress(Q, K, np.array([0, n]), tau=0.7, B=B)
    for b in range(len(part.brow_I)):
        I = int(part.brow_I[b])
        rows = min(n, (I + 1) * B) - I * B
        blocks = {int(part.block_idx[t]): part.probs[t] for t in range(part.block_ptr[b], part.block_ptr[b + 1])}
        Abar, _ = mo.renormalise(mo.mix_heads(mo.gather_row_probs(blocks, B, rows, 0, n)[0], W2))
        assert np.allclose(Abar.sum(axis=2), 1.0, atol=1e-13)


def test_mix_heads_scalar_brute_force():
    rng = np.random.default_rng(10)
    P = rng.random((5, 3, 7))
    W = rng.standard_normal((4, 5))
    got = mo.mix_heads(P, W)
    for g in range(4):
        for i in range(3):
            for j in range(7):
                assert abs(got[g, i, j] - sum(W[g, h] * P[h, i, j] for h in range(5))) < 1e-14


def test_constant_v_rows_give_that_row():
    """I7: V[j, kv, :] = v for every j  ->  O[i, g, :] = v for any tau and W."""
    rng = np.random.default_rng(11)
    H, n, d, B = 4, 60, 8, 16
    Q, K = _rand_qk(rng, H, n, d)
    v = rng.standard_normal((2, d))
    V = np.broadcast_to(v[None], (n, 2, d)).copy()
    bsr = mo.compress(Q, K, np.array([0, n]), tau=0.6, B=B)
    W = rng.dirichlet(np.full(H, 0.5), size=4)
    kv = [0, 0, 1, 1]
    O = mo.retrieve(bsr, W, V, kv)
    for g in range(4):
        assert np.allclose(O[:, g, :], v[kv[g]], atol=1e-13)


def test_v_readout_exposes_mixed_map():
    """I8: V[j, kv, c] = [j == j0 + c] makes O[i, g, c] equal Abar[g, i, j0 + c]."""
    rng = np.random.default_rng(12)
    H, n, d, B = 3, 48, 16, 16
    Q, K = _rand_qk(rng, H, n, d)
    W = rng.dirichlet(np.full(H, 0.5), size=2)
    bsr = mo.compress(Q, K, np.array([0, n]), tau=0.7, B=B)
    for j0 in [0, 16, 32]:
        V = np.zeros((n, 1, d))
        for c in range(d):
            V[j0 + c, 0, c] = 1.0
        O = mo.retrieve(bsr, W, V, [0, 0])
        for b in range(len(bsr.brow_I)):
            I = int(bsr.brow_I[b])
            rows = min(n, (I + 1) * B) - I * B
            blocks = {int(bsr.block_idx[t]): bsr.probs[t] for t in range(bsr.block_ptr[b], bsr.block_ptr[b + 1])}
            # dense mixed map over all keys of this block row, zero at dropped blocks
            dense = np.zeros((2, rows, n))
            for J, p in blocks.items():
                for g in range(2):
                    for h in range(H):
                        dense[g, :, J * B:(J + 1) * B] += W[g, h] * p[h, :rows, :]
            dense /= dense.sum(axis=2, keepdims=True)
            for g in range(2):
                assert np.allclose(O[I * B: I * B + rows, g, :], dense[g, :, j0:j0 + d], atol=1e-14)


def test_sender_head_permutation_invariance():
    rng = np.random.default_rng(13)
    H, n, d, B = 5, 40, 8, 8
    Q, K = _rand_qk(rng, H, n, d)
    V = rng.standard_normal((n, 2, d))
    W = rng.standard_normal((3, H)) + 1.0
    perm = rng.permutation(H)
    a = mo.compress(Q, K, np.array([0, n]), tau=0.75, B=B)
    b = mo.compress(Q[perm], K[perm], np.array([0, n]), tau=0.75, B=B)
    Oa = mo.retrieve(a, W, V, [0, 1, 1])
    Ob = mo.retrieve(b, W[:, perm], V, [0, 1, 1])
    assert np.array_equal(a.block_idx, b.block_idx)
    assert np.allclose(Oa, Ob, atol=1e-12)


def test_one_hot_w_is_block_sparse_attention_of_one_sender_head():
    """W[g] = e_{h(g)} reduces retrieve to head h(g)'s attention restricted to the kept blocks."""
    rng = np.random.default_rng(14)
    H, n, d, B = 3, 56, 8, 8
    Q, K = _rand_qk(rng, H, n, d)
    V = rng.standard_normal((n, 1, d))
    hsel = [2, 0]
    W = np.zeros((2, H))
    for g, h in enumerate(hsel):
        W[g, h] = 1.0
    bsr = mo.compress(Q, K, np.array([0, n]), tau=0.6, B=B, keep_exact=True)
    O = mo.retrieve(bsr, W, V, [0, 0], unrounded=True)
    for b in range(len(bsr.brow_I)):
        I = int(bsr.brow_I[b])
        keep = np.zeros(n, bool)
        for t in range(bsr.block_ptr[b], bsr.block_ptr[b + 1]):
            J = int(bsr.block_idx[t])
            keep[J * B:(J + 1) * B] = True
        for g, h in enumerate(hsel):
            rows = slice(I * B, min(n, (I + 1) * B))
            s = torch.from_numpy(Q[h, rows] @ K[h].T / math.sqrt(d))
            i_idx = torch.arange(rows.start, rows.stop)[:, None]
            mask = (torch.arange(n)[None, :] <= i_idx) & torch.from_numpy(keep)[None, :]
            p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=1).numpy()
            assert np.allclose(O[rows, g, :], p @ V[:, 0, :], atol=1e-12)


# ------------------------------------------------------------------------- varlen and paged V
def test_varlen_packed_equals_per_sequence_and_paged_equals_contiguous():
    wl = synth.WORKLOADS["varlen_14b8b"]
    lengths = [37, 64, 129, 5]
    x = synth.make_layer_inputs(wl, 3, lengths=lengths, H_s=3, H_r=4, H_kv=2, d=16)
    cu = x["cu_seqlens"]
    packed = mo.compress(x["q_s"], x["k_s"], cu, tau=0.8, B=32)
    Op = mo.retrieve(packed, x["w"], x["v_r"], x["kv_head_map"])
    for s, n in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        one = mo.compress(x["q_s"][:, a:b], x["k_s"][:, a:b], np.array([0, n]), tau=0.8, B=32)
        lo = int(packed.block_ptr[list(packed.brow_seq).index(s)])
        hi = lo + len(one.block_idx)
        assert np.array_equal(packed.block_idx[lo:hi], one.block_idx)
        assert np.array_equal(packed.probs[lo:hi], one.probs)
        Oo = mo.retrieve(one, x["w"], x["v_r"][a:b], x["kv_head_map"])
        assert np.array_equal(Op[a:b], Oo)
    table, n_pages = synth.make_page_table(lengths, 16, seed=3)
    pool = synth.page_v(x["v_r"], lengths, table, 16, n_pages)
    Og = mo.retrieve(packed, x["w"], pool, x["kv_head_map"], page_table=table, page_size=16)
    assert np.array_equal(Og, Op)


# -------------------------------------------------------------------------- dense recompute
def test_dense_causal_attention_vs_sdpa_with_gqa():
    rng = np.random.default_rng(15)
    T, Hq, Hkv, d = 70, 6, 2, 8
    lengths = [30, 40]
    Q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    kv = [g // 3 for g in range(Hq)]
    O = mo.dense_causal_attention(Q, K, V, np.array([0, 30, 70]), kv)
    for a, b in [(0, 30), (30, 70)]:
        q = torch.from_numpy(Q[a:b].transpose(1, 0, 2).copy())
        k = torch.from_numpy(K[a:b].transpose(1, 0, 2).copy()).repeat_interleave(3, dim=0)
        v = torch.from_numpy(V[a:b].transpose(1, 0, 2).copy()).repeat_interleave(3, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        assert np.allclose(O[a:b], ref.numpy().transpose(1, 0, 2), atol=1e-12)


# ------------------------------------------------------------------------------- layer map
def test_layer_map_rounds_linear_depth_map():
    pi = mo.layer_map(28, 36, 2)
    assert pi[:2] == [-1, -1]
    for l in range(2, 28):
        x = l * 35 / 27
        assert abs(pi[l] - x) <= 0.5 and 0 <= pi[l] <= 35
    assert pi[27] == 35 and pi == sorted(pi)
    assert mo.layer_map(5, 5, 0) == [0, 1, 2, 3, 4]
    assert mo.layer_map(3, 6, 0) == [0, 3, 5]            # 2.5 rounds up
    assert mo.layer_map(1, 4, 0) == [0]


# --------------------------------------------------------------- planted mistakes are caught
def _catches(monkeypatch, name, bad, pin):
    with monkeypatch.context() as m:
        m.setattr(mo, name, bad)
        with pytest.raises(AssertionError):
            pin()


# ------------------------------------------------------------------ variants (next row 4 of the scope)
def test_per_head_selection_reduces_to_shared_selection_with_one_head():
    rng = np.random.default_rng(21)
    q, k = _rand_qk(rng, 1, 150, 16)
    cu = [0, 150]
    a = oracle.compress(q, k, cu, 0.6, 32)
    b = oracle.compress(q, k, cu, 0.6, 32, per_head_select=True)
    assert np.array_equal(a.block_idx, b.block_idx) and np.array_equal(a.probs, b.probs)
    assert np.array_equal(a.row_kept_mass, b.row_kept_mass)


def test_per_head_selection_invariants_by_brute_force():
    """Each head's own set is the brute-force selection of its own masses (total = rows); the
    store keeps their union and a head's probabilities vanish outside its own set."""
    rng = np.random.default_rng(22)
    q, k = _rand_qk(rng, 3, 170, 16)
    cu = [0, 170]
    B, tau = 32, 0.55
    st = oracle.compress(q, k, cu, tau, B, per_head_select=True)
    full = oracle.compress(q, k, cu, 1.0, B)                 # every block, exact per-head values
    for b, r in enumerate(st.rows):
        I, rows = r["I"], r["rows"]
        union = set()
        for h in range(3):
            A, _ = mo.attention_rows(q[h].astype(np.float64), k[h].astype(np.float64), I * B, I * B + rows)
            masses = np.array([A[:, J * B: min(170, (J + 1) * B)].sum() for J in range(I + 1)])
            own = _brute_select(masses, I, float(rows), tau)
            union |= set(own)
            lo, hi = int(st.block_ptr[b]), int(st.block_ptr[b + 1])
            for t in range(lo, hi):
                J = int(st.block_idx[t])
                ref = full.probs[int(full.block_ptr[b]) + J][h]
                assert np.array_equal(st.probs[t][h], ref if J in own else np.zeros_like(ref))
        assert sorted(union) == list(st.block_idx[int(st.block_ptr[b]): int(st.block_ptr[b + 1])])


def test_per_head_normalisation():
    rng = np.random.default_rng(23)
    q, k = _rand_qk(rng, 2, 140, 16)
    cu = [0, 140]
    # every block kept: each head's kept mass is exactly 1, so nothing changes
    a = oracle.compress(q, k, cu, 1.0, 32)
    b = oracle.compress(q, k, cu, 1.0, 32, per_head_norm=True)
    assert np.array_equal(a.probs, b.probs)
    # otherwise each head's stored row sums to 1 up to its bf16 roundings, and the values are the
    # exact map divided by the head's exact kept mass
    st = oracle.compress(q, k, cu, 0.5, 32, per_head_norm=True, keep_exact=True)
    plain = oracle.compress(q, k, cu, 0.5, 32, keep_exact=True)
    assert np.array_equal(st.block_idx, plain.block_idx)
    for b, r in enumerate(st.rows):
        lo, hi = int(st.block_ptr[b]), int(st.block_ptr[b + 1])
        rows = r["rows"]
        s = st.probs[lo:hi, :, :rows].sum(axis=(0, 3))                       # [H, rows]
        assert np.all(np.abs(s - 1.0) <= 2.0 ** -8)
        mass = plain.exact[lo:hi, :, :rows].sum(axis=(0, 3))                 # exact kept mass
        ratio = plain.exact[lo:hi, :, :rows] / mass[None, :, :, None]
        assert np.allclose(st.exact[lo:hi, :, :rows], ratio, rtol=1e-12, atol=0)


def test_cross_layer_retrieve_reductions():
    """One layer is the single-layer retrieve; two copies of one store with W split between them
    give the retrieve with the whole W; two layers with one-hot weights on one layer's heads give
    that layer's retrieve restricted to the union of blocks (zeros elsewhere do not count)."""
    x = synth.make_layer_inputs(synth.WORKLOADS["tiny"], 24, lengths=[160], H_s=4, H_r=3, H_kv=3, d=16)
    a = oracle.compress(x["q_s"], x["k_s"], x["cu_seqlens"], 0.6, 32)
    W = x["w"].astype(np.float64)                # split exactly: 0.25 W + 0.75 W == W in fp64
    ref = oracle.retrieve(a, W, x["v_r"], x["kv_head_map"])
    assert np.allclose(oracle.retrieve_layers([a], [W], x["v_r"], x["kv_head_map"]), ref, rtol=1e-12, atol=1e-12)
    split = oracle.retrieve_layers([a, a], [0.25 * W, 0.75 * W], x["v_r"], x["kv_head_map"])
    assert np.allclose(split, ref, rtol=1e-12, atol=1e-12)
    y = synth.make_layer_inputs(synth.WORKLOADS["tiny"], 25, lengths=[160], H_s=4, H_r=3, H_kv=3, d=16)
    b = oracle.compress(y["q_s"], y["k_s"], y["cu_seqlens"], 0.6, 32)
    only_a = oracle.retrieve_layers([a, b], [W, np.zeros_like(W)], x["v_r"], x["kv_head_map"])
    assert np.allclose(only_a, ref, rtol=1e-12, atol=1e-12)
    both = oracle.retrieve_layers([a, b], [W, W], x["v_r"], x["kv_head_map"])
    assert not np.allclose(both, ref)            # the second layer does contribute


def test_pins_catch_planted_mistakes(monkeypatch):
    orig_rows = mo.attention_rows
    orig_mix = mo.mix_heads
    orig_apply = mo.apply_v
    orig_select = mo.select_blocks

    def no_scale(q, k, r0, r1):                          # dropped 1/sqrt(d)
        return orig_rows(np.asarray(q) * math.sqrt(q.shape[1]), k, r0, r1)

    def no_causal_shift(q, k, r0, r1):                   # off-by-one causal mask
        A, lse = orig_rows(q, k, r0, r1)
        return np.roll(A, 1, axis=1), lse

    def transposed_w(P, W):                              # W used transposed
        return orig_mix(P, np.asarray(W).T[: np.asarray(W).shape[0], : np.asarray(W).shape[1]])

    def shifted_keys(Abar, keys, V, kv_head_map, *a, **kw):   # keys off by one
        return orig_apply(Abar, np.minimum(keys + 1, V.shape[0] - 1), V, kv_head_map, *a, **kw)

    def no_forced_diag(M_row, I, T_I, tau):             # diagonal block not forced
        r = orig_select(M_row, I, T_I, tau)
        if I > 0 and tau < 1.0 and I in r["kept"]:
            r = dict(r, kept=[J for J in r["kept"] if J != I])
        return r

    _catches(monkeypatch, "attention_rows", no_scale, test_attention_rows_vs_library_routines)
    _catches(monkeypatch, "attention_rows", no_causal_shift, test_block_masses_brute_force_and_conservation)
    _catches(monkeypatch, "mix_heads", transposed_w, test_sender_head_permutation_invariance)
    _catches(monkeypatch, "apply_v", shifted_keys, test_v_readout_exposes_mixed_map)
    _catches(monkeypatch, "select_blocks", no_forced_diag, test_selection_invariants)
