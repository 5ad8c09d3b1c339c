"""fp64 CPU oracle for MapFlow's compress and fused-retrieve stages.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never imports this.

The pages describe the method in prose only; this file writes out the plainest definitions that
prose supports, in float64 with numpy, one step after another:

  scores -> causal softmax map -> explicit block sums -> sorted block selection ->
  bf16 kept probabilities and kept row mass -> explicit sum over sender heads of W times P ->
  row renormalisation -> matmul with the receiver's V.

Inputs are the exact tensors handed to the GPU (bf16 or fp32 values promoted to fp64).
Readings taken where the pages are silent are marked "Reading:" and listed in the design notes.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------------------------
# bf16 rounding of the stored probabilities
# ----------------------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even, directly from fp64.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent range.  Normal
    values: write x = m * 2**e with 0.5 <= |m| < 1 and round m * 2**8 to an integer (ties to
    even).  Below 2**-126 the spacing is fixed at 2**-133 (subnormals).  Reading: the block store
    holds "probs bf16"; the pages fix no rounding mode, round-to-nearest-even is the IEEE default.
    """
    x = np.asarray(x, dtype=F64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    m, e = np.frexp(np.where(finite, x, 0.0))
    out[...] = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = finite & (np.abs(x) < 2.0 ** -126)
    out[sub] = np.ldexp(np.rint(np.ldexp(x[sub], 133)), -133)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    # values that round past the largest finite bf16 overflow to infinity
    big = finite & (np.abs(out) > max_bf16)
    out[big] = np.copysign(np.inf, x[big])
    out[~finite] = x[~finite]
    return out


# ----------------------------------------------------------------------------------------------
# O1-O3: scores, row logsumexp and the causal softmax attention map
# ----------------------------------------------------------------------------------------------
def attention_rows(q: np.ndarray, k: np.ndarray, r0: int, r1: int):
    """Rows r0..r1-1 of one head's causal softmax attention map within one sequence.

    [MapFlow开源, 不传 KV Cache 改传注意力关系] and [Reuses Attention, attention-map section]:
    the map records, for each token, how much attention it gives to each other token.  Reading:
    the standard scaled dot product s_ij = q_i . k_j / sqrt(d) with a causal mask (j <= i);
    q and k are the sender's post-RoPE queries and keys.

    q, k: [n, d] float64 for one head of one sequence.  Returns (A, lse) with A [r1-r0, r1]
    (zero above the diagonal) and lse [r1-r0] the natural-log row logsumexp.
    """
    q = np.asarray(q[r0:r1], dtype=F64)
    k = np.asarray(k[:r1], dtype=F64)
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d)                                  # [rows, r1]
    i_idx = np.arange(r0, r1)[:, None]
    j_idx = np.arange(r1)[None, :]
    causal = j_idx <= i_idx
    s = np.where(causal, s, -np.inf)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    A = np.where(causal, np.exp(s - lse[:, None]), 0.0)
    return A, lse


# ----------------------------------------------------------------------------------------------
# O5: block selection by cumulative attention mass
# ----------------------------------------------------------------------------------------------
def select_blocks(M_row: np.ndarray, I: int, T_I: float, tau: float) -> dict:
    """Kept block columns of block row I.

    [MapFlow开源, 只存重要的:块稀疏压缩] and [Reuses Attention, first component]: cut the map into
    regular 2-D blocks and keep the high-attention ones, chosen by cumulative attention
    probability, after first computing block-level statistics.

    Readings: the sink block (column 0) and the diagonal block (column I) are always kept; the
    remaining columns are taken in order of descending mass (ties: lower column first) until the
    cumulative kept mass reaches tau * T_I, where T_I = (sender heads) x (rows in the block row)
    is the total mass of the block row; the check happens before each addition, so the block that
    crosses the threshold is kept.  tau >= 1 keeps every causal block.

    Returns {"kept": ascending list, "last_mass": mass of the last block added by the walk (None
    when only forced blocks are kept), "cum_before_last": cumulative mass before that block,
    "cum": final cumulative mass}.
    """
    if tau >= 1.0:
        return {"kept": list(range(I + 1)), "last_mass": None, "cum_before_last": None,
                "cum": float(np.sum(M_row[: I + 1]))}
    forced = sorted({0, I})
    c = 0.0
    for J in forced:
        c += float(M_row[J])
    rest = sorted((J for J in range(I + 1) if J not in forced), key=lambda J: (-float(M_row[J]), J))
    kept = set(forced)
    target = tau * T_I
    last_mass = None
    cum_before_last = None
    for J in rest:
        if c >= target:
            break
        cum_before_last = c
        kept.add(J)
        c += float(M_row[J])
        last_mass = float(M_row[J])
    return {"kept": sorted(kept), "last_mass": last_mass, "cum_before_last": cum_before_last,
            "cum": c}


# ----------------------------------------------------------------------------------------------
# O4-O7 for one block row: block masses, selection, bf16 probs, kept row mass
# ----------------------------------------------------------------------------------------------
def block_masses(Q: np.ndarray, K: np.ndarray, seq_start: int, seq_len: int, I: int, B: int,
                 per_head: bool = False):
    """Block-level statistics of block row I of one sequence: the first stage of the staged
    compression in [MapFlow开源, 只存重要的:块稀疏压缩].

    M[J] = sum_h sum_{i in I} sum_{j in J} A[h, i, j] for J = 0..I (explicit block sums over the
    causal softmax map of every sender head); also returns lse [H_s, rows].  With ``per_head``,
    M[h, J] is the same sum without the sum over h.
    """
    H_s = Q.shape[0]
    r0 = I * B
    r1 = min(seq_len, (I + 1) * B)
    rows = r1 - r0
    Mh = np.zeros((H_s, I + 1), dtype=F64)
    lse = np.zeros((H_s, rows), dtype=F64)
    for h in range(H_s):
        q = Q[h, seq_start: seq_start + seq_len]
        k = K[h, seq_start: seq_start + seq_len]
        A, lse[h] = attention_rows(q, k, r0, r1)
        for J in range(I + 1):
            c0 = J * B
            c1 = min(seq_len, (J + 1) * B)
            Mh[h, J] = A[:, c0:c1].sum()
    if per_head:
        return Mh, lse
    M = np.zeros(I + 1, dtype=F64)
    for h in range(H_s):
        M += Mh[h]
    return M, lse


def block_row_compress(Q: np.ndarray, K: np.ndarray, seq_start: int, seq_len: int, I: int,
                       B: int, tau: float, keep_exact: bool = False, per_head_select: bool = False,
                       per_head_norm: bool = False) -> dict:
    """Compress block row I of one sequence (all sender heads).

    Q, K: [H_s, T, d] (the packed batch); the sequence occupies tokens
    [seq_start, seq_start + seq_len).  Two passes over the heads, as the staged compression in
    [MapFlow开源, 只存重要的:块稀疏压缩] describes (statistics first, then the kept blocks):

    pass 1  M[J] = sum_h sum_{i in I} sum_{j in J} A[h, i, j]   (explicit block sums)
    select  as ``select_blocks``
    pass 2  probs[J][h, r, c] = bf16(A[h, I*B + r, J*B + c]) for kept J (zero outside the valid /
            causal region); row_kept_mass[h, r] = sum over kept J and c of probs (in fp64).

    Variants the wording allows ([MapFlow 方案, 二] names cross-layer and cross-head mapping;
    [MapFlow开源, the head-mapping bullet] mixes sender heads), off by default:
    per_head_select  every sender head selects its own blocks from its own masses M[h, J] with
                     total mass ``rows`` (same forced blocks, order and stopping rule); the store
                     keeps the union of the heads' sets and a head's probabilities are 0 in the
                     blocks it did not select
    per_head_norm    each head's row is divided by that head's mass over its kept blocks (exact)
                     before the bf16 rounding, so a head's stored row sums to about 1
    """
    H_s = Q.shape[0]
    r0 = I * B
    r1 = min(seq_len, (I + 1) * B)
    rows = r1 - r0
    if per_head_select:
        Mh, lse = block_masses(Q, K, seq_start, seq_len, I, B, per_head=True)
        sel_h = [select_blocks(Mh[h], I, float(rows), tau) for h in range(H_s)]
        head_kept = [set(sh["kept"]) for sh in sel_h]
        kept = sorted(set().union(*head_kept))
        M = Mh.sum(axis=0)
        sel = {"kept": kept, "per_head": sel_h}
        T_I = float(H_s * rows)
    else:
        M, lse = block_masses(Q, K, seq_start, seq_len, I, B)
        T_I = float(H_s * rows)
        sel = select_blocks(M, I, T_I, tau)
        kept = sel["kept"]
        head_kept = [set(kept) for _ in range(H_s)]
    probs = {J: np.zeros((H_s, B, B), dtype=F64) for J in kept}
    exact = {J: np.zeros((H_s, B, B), dtype=F64) for J in kept} if keep_exact else None
    for h in range(H_s):
        q = Q[h, seq_start: seq_start + seq_len]
        k = K[h, seq_start: seq_start + seq_len]
        A, _ = attention_rows(q, k, r0, r1)
        if per_head_norm:
            mass = np.zeros(rows, dtype=F64)
            for J in sorted(head_kept[h]):
                mass += A[:, J * B: min(seq_len, (J + 1) * B)].sum(axis=1)
            A = A / mass[:, None]
        for J in kept:
            if J not in head_kept[h]:
                continue
            c0 = J * B
            c1 = min(seq_len, (J + 1) * B)
            tile = A[:, c0:c1]
            probs[J][h, :rows, : c1 - c0] = bf16_round(tile)
            if keep_exact:
                exact[J][h, :rows, : c1 - c0] = tile
    row_kept_mass = np.zeros((H_s, rows), dtype=F64)
    for J in kept:
        row_kept_mass += probs[J][:, :rows, :].sum(axis=2)
    return {"I": I, "rows": rows, "tok0": seq_start + r0, "M": M, "T_I": T_I, "sel": sel,
            "kept": kept, "probs": probs, "exact": exact, "row_kept_mass": row_kept_mass,
            "lse": lse}


@dataclasses.dataclass
class OracleBSR:
    """Block-sparse store in canonical layout: probs [nnzb, H_s, B, B] (fp64 holding bf16 values)."""
    B: int
    H_s: int
    cu_seqlens: np.ndarray
    brow_seq: np.ndarray        # [n_brow] sequence of each block row
    brow_I: np.ndarray          # [n_brow] block row index within its sequence
    block_ptr: np.ndarray       # [n_brow + 1]
    block_idx: np.ndarray       # [nnzb] block column within the sequence, ascending per row
    probs: np.ndarray           # [nnzb, H_s, B, B]
    row_kept_mass: np.ndarray   # [H_s, T]
    lse: np.ndarray             # [H_s, T]
    rows: list                  # per block row: the dict returned by block_row_compress
    exact: np.ndarray | None = None   # unrounded probabilities of the kept blocks, same layout


def compress(Q, K, cu_seqlens, tau: float, B: int, keep_exact: bool = False,
             per_head_select: bool = False, per_head_norm: bool = False) -> OracleBSR:
    """mf_compress's definition over a packed batch: every sequence and block row in turn
    (``per_head_select`` / ``per_head_norm``: the variants of ``block_row_compress``).

    Varlen reading: each sequence has its own block grid starting at its first token, and its
    block column 0 is its own sink block.
    """
    Q = np.asarray(Q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    H_s, T = Q.shape[0], Q.shape[1]
    brow_seq, brow_I, ptr, idx, probs, exact, rows = [], [], [0], [], [], [], []
    rkm = np.zeros((H_s, T), dtype=F64)
    lse = np.zeros((H_s, T), dtype=F64)
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        for I in range((n + B - 1) // B):
            r = block_row_compress(Q, K, int(cu[s]), n, I, B, tau, keep_exact, per_head_select, per_head_norm)
            rows.append(r)
            brow_seq.append(s)
            brow_I.append(I)
            for J in r["kept"]:
                idx.append(J)
                probs.append(r["probs"][J])
                if keep_exact:
                    exact.append(r["exact"][J])
            ptr.append(len(idx))
            rkm[:, r["tok0"]: r["tok0"] + r["rows"]] = r["row_kept_mass"]
            lse[:, r["tok0"]: r["tok0"] + r["rows"]] = r["lse"]
    empty = np.zeros((0, H_s, B, B), dtype=F64)
    return OracleBSR(
        B=B, H_s=H_s, cu_seqlens=cu.copy(), brow_seq=np.array(brow_seq, np.int64),
        brow_I=np.array(brow_I, np.int64), block_ptr=np.array(ptr, np.int64),
        block_idx=np.array(idx, np.int64), probs=np.stack(probs) if probs else empty,
        row_kept_mass=rkm, lse=lse, rows=rows,
        exact=(np.stack(exact) if exact else empty) if keep_exact else None)


# ----------------------------------------------------------------------------------------------
# O8-O10: fused retrieve (head mix, renormalise, multiply by the receiver's V)
# ----------------------------------------------------------------------------------------------
def _v_rows(V, tokens: np.ndarray, kv: int, page_table=None, page_size: int = 16,
            seq: int = 0, seq_start: int = 0) -> np.ndarray:
    """V rows of kv head ``kv`` for packed token indices (contiguous [T, H_kv, d] or paged)."""
    if page_table is None:
        return np.asarray(V[tokens, kv, :], dtype=F64)
    local = tokens - seq_start
    pages = np.asarray(page_table)[seq, local // page_size]
    return np.asarray(V[pages, local % page_size, kv, :], dtype=F64)


def gather_row_probs(probs_by_J: dict, B: int, rows: int, seq_start: int, seq_len: int):
    """Concatenate the kept blocks of one block row: (P [H_s, rows, K], packed key tokens [K])."""
    P_parts, key_parts = [], []
    for J in sorted(probs_by_J):
        c0 = J * B
        c1 = min(seq_len, (J + 1) * B)
        P_parts.append(np.asarray(probs_by_J[J], dtype=F64)[:, :rows, : c1 - c0])
        key_parts.append(np.arange(seq_start + c0, seq_start + c1))
    return np.concatenate(P_parts, axis=2), np.concatenate(key_parts)


def mix_heads(P: np.ndarray, W) -> np.ndarray:
    """Ahat[g, i, j] = sum_h W[g, h] P[h, i, j], written as an explicit sum over sender heads.

    [MapFlow开源, 改传注意力关系]: head mapping is a learned set of linear-combination weights that
    merges sender heads into receiver heads; [MapFlow开源, 融合内核执行] does this combination on
    chip.  Reading: one real [H_r, H_s] matrix per mapped receiver layer, no bias.
    """
    W = np.asarray(W, dtype=F64)
    H_r, H_s = W.shape
    Ahat = np.zeros((H_r,) + P.shape[1:], dtype=F64)
    for g in range(H_r):
        for h in range(H_s):
            Ahat[g] += W[g, h] * P[h]
    return Ahat


def renormalise(Ahat: np.ndarray):
    """Reading: each mixed row is divided by its sum over the kept keys.  Returns (Abar, den)."""
    den = Ahat.sum(axis=2)
    return Ahat / den[:, :, None], den


def apply_v(Abar: np.ndarray, keys: np.ndarray, V, kv_head_map, page_table=None,
            page_size: int = 16, seq: int = 0, seq_start: int = 0) -> np.ndarray:
    """O[i, g, :] = sum_j Abar[g, i, j] V[kv(g), key_j, :], a plain matmul with the receiver's V.

    [MapFlow开源, 改传注意力关系] and [Reuses Attention, attention-map section]: the receiver keeps
    its own Value representation.  Returns [rows, H_r, d].
    """
    H_r, rows = Abar.shape[0], Abar.shape[1]
    out = np.zeros((rows, H_r, V.shape[-1]), dtype=F64)
    for g in range(H_r):
        Vg = _v_rows(V, keys, int(kv_head_map[g]), page_table, page_size, seq, seq_start)
        out[:, g, :] = Abar[g] @ Vg
    return out


def retrieve_block_row(probs_by_J: dict, B: int, rows: int, tok0: int, seq: int, seq_start: int,
                       seq_len: int, W, V, kv_head_map, page_table=None,
                       page_size: int = 16) -> np.ndarray:
    """Receiver output rows of one block row, [rows, H_r, d].

    [MapFlow开源, 算得省的:融合内核执行] and [Reuses Attention, third component]: read the kept
    sparse blocks, combine the sender heads linearly into receiver heads, then multiply by the
    receiver's own V and accumulate, with no reconstructed dense matrix.  The steps:
    ``gather_row_probs`` -> ``mix_heads`` -> ``renormalise`` -> ``apply_v``.
    """
    P, keys = gather_row_probs(probs_by_J, B, rows, seq_start, seq_len)
    Abar, _ = renormalise(mix_heads(P, W))
    return apply_v(Abar, keys, V, kv_head_map, page_table, page_size, seq, seq_start)


def retrieve(bsr: OracleBSR, W, V, kv_head_map, page_table=None, page_size: int = 16,
             unrounded: bool = False) -> np.ndarray:
    """O_r [T, H_r, d] for a whole block-sparse store (mf_retrieve's definition).

    ``unrounded`` uses the exact fp64 map of the kept blocks instead of the bf16 probs (used only
    by the invariant checks that compare against dense attention).
    """
    W = np.asarray(W, dtype=F64)
    H_r = W.shape[0]
    T = bsr.row_kept_mass.shape[1]
    d = V.shape[-1]
    O = np.zeros((T, H_r, d), dtype=F64)
    src = bsr.exact if unrounded else bsr.probs
    cu = bsr.cu_seqlens
    for b in range(len(bsr.brow_seq)):
        s = int(bsr.brow_seq[b])
        I = int(bsr.brow_I[b])
        n = int(cu[s + 1] - cu[s])
        rows = min(n, (I + 1) * bsr.B) - I * bsr.B
        tok0 = int(cu[s]) + I * bsr.B
        lo, hi = int(bsr.block_ptr[b]), int(bsr.block_ptr[b + 1])
        blocks = {int(bsr.block_idx[t]): src[t] for t in range(lo, hi)}
        O[tok0: tok0 + rows] = retrieve_block_row(blocks, bsr.B, rows, tok0, s, int(cu[s]), n, W,
                                                  V, kv_head_map, page_table, page_size)
    return O


def retrieve_layers(bsrs, Ws, V, kv_head_map) -> np.ndarray:
    """One receiver layer from the stores of several sender layers (contiguous V only).

    [MapFlow 方案, 二]: the mapping is linear across layers and across heads.  Reading: the mixed
    map of receiver head g is sum over layers l and sender heads h of W_l[g, h] P_l[h], with P_l
    zero outside layer l's kept blocks; the row is renormalised over the union of kept blocks and
    multiplied by the receiver's V, as for one layer.
    """
    first = bsrs[0]
    B = first.B
    cu = first.cu_seqlens
    Ws = [np.asarray(W, dtype=F64) for W in Ws]
    H_r = Ws[0].shape[0]
    T = first.row_kept_mass.shape[1]
    O = np.zeros((T, H_r, V.shape[-1]), dtype=F64)
    for b in range(len(first.brow_seq)):
        s = int(first.brow_seq[b])
        I = int(first.brow_I[b])
        n = int(cu[s + 1] - cu[s])
        rows = min(n, (I + 1) * B) - I * B
        tok0 = int(cu[s]) + I * B
        union = sorted({int(bsr.block_idx[t]) for bsr in bsrs
                        for t in range(int(bsr.block_ptr[b]), int(bsr.block_ptr[b + 1]))})
        Ahat = None
        for bsr, W in zip(bsrs, Ws):
            lo, hi = int(bsr.block_ptr[b]), int(bsr.block_ptr[b + 1])
            blocks = {int(bsr.block_idx[t]): bsr.probs[t] for t in range(lo, hi)}
            full = {J: blocks.get(J, np.zeros((bsr.H_s, B, B), dtype=F64)) for J in union}
            P, keys = gather_row_probs(full, B, rows, int(cu[s]), n)
            part = mix_heads(P, W)
            Ahat = part if Ahat is None else Ahat + part
        Abar, _ = renormalise(Ahat)
        O[tok0: tok0 + rows] = apply_v(Abar, keys, V, kv_head_map)
    return O


# ----------------------------------------------------------------------------------------------
# O11: dense causal attention for the recomputed receiver layers
# ----------------------------------------------------------------------------------------------
def dense_causal_attention(Q, K, V, cu_seqlens, kv_head_map) -> np.ndarray:
    """softmax(Q K^T / sqrt(d), causal) V per query head, with query head g reading KV head
    kv_head_map[g].

    [Reuses Attention, attention-map section]: the receiver first computes its early layers
    normally (partial recomputation, also named in [Abstract]).  Q [T, H_q, d], K, V [T, H_kv, d].
    """
    Q = np.asarray(Q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    T, H_q, d = Q.shape
    O = np.zeros((T, H_q, d), dtype=F64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for g in range(H_q):
            kv = int(kv_head_map[g])
            A, _ = attention_rows(Q[a:b, g], K[a:b, kv], 0, b - a)
            O[a:b, g] = A @ V[a:b, kv]
    return O


# ----------------------------------------------------------------------------------------------
# Layer mapping
# ----------------------------------------------------------------------------------------------
def layer_map(n_recv: int, n_send: int, R: int) -> list[int]:
    """Receiver layer -> sender layer, -1 for the first R receiver layers (recomputed densely).

    [MapFlow开源, 改传注意力关系]: a sender layer's map is assigned to a suitable receiver layer.
    Reading: spread the receiver's depth linearly over the sender's,
    pi(l) = round(l * (n_send - 1) / (n_recv - 1)), halves rounded up, computed exactly.
    """
    out = []
    for l in range(n_recv):
        if l < R:
            out.append(-1)
            continue
        if n_recv == 1:
            out.append(0)
            continue
        x = Fraction(l * (n_send - 1), n_recv - 1)
        out.append(int(math.floor(x + Fraction(1, 2))))
    return out
