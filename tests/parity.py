"""Comparison rules between the HIP path and the oracle (shared by the GPU tests).

Tolerances:
* kept-block sets: identical, except at ties within 1e-6 relative mass (rule below);
* kept probabilities: |p_gpu - A| <= ulp_bf16(A) + 1e-6 against the exact fp64 map;
* outputs: relative Frobenius error <= 1e-3 and max absolute error <= 5e-3 against the oracle
  run on the same bf16 blocks.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TIE = 1e-6
O_REL_FRO = 1e-3
O_MAX_ABS = 5e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str | torch.dtype = torch.float32) -> torch.Tensor:
    if dtype == "bf16":
        dtype = torch.bfloat16
    elif dtype == "f32":
        dtype = torch.float32
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dtype)
    return t.to("cuda")


def ulp_bf16(a: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.frexp(np.where(a > 0, a, 1.0))[1]       # a = m 2^e, m in [0.5, 1)
    u = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.where(a > 0, u, 0.0)


def sets_agree(gpu_kept: list[int], row: dict, tau: float) -> tuple[bool, str]:
    """Acceptance rule for one block row: equal sets pass; otherwise every difference must be a
    tie within 1e-6 relative mass of the oracle's marginal block, and a size difference needs the
    oracle's cumulative mass at the boundary within 1e-6 T_I of the target."""
    S_g, S_o = set(gpu_kept), set(row["kept"])
    if S_g == S_o:
        return True, ""
    M, T_I, sel = row["M"], row["T_I"], row["sel"]
    target = tau * T_I
    forced = {0, row["I"]}
    if not forced <= S_g:
        return False, "forced block missing"
    m_star = sel["last_mass"]
    if m_star is None:
        c_forced = sum(M[J] for J in forced)
        ok = abs(c_forced - target) <= TIE * T_I
        return ok, f"oracle kept only forced blocks; gap {abs(c_forced - target) / T_I:.2e}"
    for J in S_g - S_o:
        if M[J] < m_star * (1 - TIE):
            return False, f"extra block {J} mass {M[J]:.6g} < marginal {m_star:.6g}"
    for J in S_o - S_g:
        if M[J] > m_star * (1 + TIE):
            return False, f"missing block {J} mass {M[J]:.6g} > marginal {m_star:.6g}"
    if len(S_g) != len(S_o):
        gap = min(abs(sel["cum_before_last"] - target), abs(sel["cum"] - target)) / T_I
        if gap > TIE:
            return False, f"size differs with boundary gap {gap:.2e}"
    return True, "tie"


def out_errors(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    got = np.asarray(got, dtype=np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(got - ref).max()) if got.size else 0.0
    return rel, mx


def assert_out_close(got, ref, what: str):
    rel, mx = out_errors(got, ref)
    say(f"  {what}: rel_fro={rel:.3e} max_abs={mx:.3e}")
    assert rel <= O_REL_FRO and mx <= O_MAX_ABS, f"{what}: rel_fro {rel:.3e}, max_abs {mx:.3e}"


def dense_maps(Q: np.ndarray, K: np.ndarray, cu) -> list:
    """Exact fp64 maps per sequence and head (small cases only): maps[s][h] = A [n, n]."""
    out = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            out.append([])
            continue
        out.append([oracle.attention_rows(Q[h, a:b].astype(np.float64), K[h, a:b].astype(np.float64), 0, b - a)[0]
                    for h in range(Q.shape[0])])
    return out


def brow_table(cu, B):
    """(seq, I) of every packed block row."""
    rows = []
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        rows += [(s, I) for I in range((n + B - 1) // B)]
    return rows


def gpu_store_for_oracle(host: dict, cu, B: int, H_s: int):
    """The GPU's downloaded store (``BlockStore.to_host()``) as an ``oracle.OracleBSR``, so that
    ``oracle.retrieve`` runs on exactly the kept blocks and bf16 probabilities the GPU stored."""
    table = brow_table(cu, B)
    return oracle.OracleBSR(
        B=B, H_s=H_s, cu_seqlens=np.asarray(cu), brow_seq=np.array([s for s, _ in table], dtype=np.int64),
        brow_I=np.array([I for _, I in table], dtype=np.int64), block_ptr=host["block_ptr"],
        block_idx=host["block_idx"], probs=host["probs"], row_kept_mass=host["row_kept_mass"],
        lse=None, rows=[])


def check_selection(host: dict, ref, tau: float, B: int) -> int:
    """Every block row's kept set against the oracle's (tie rule); returns the excused rows."""
    excused = 0
    for b in range(len(host["block_ptr"]) - 1):
        got = host["block_idx"][host["block_ptr"][b]:host["block_ptr"][b + 1]].tolist()
        ok, why = sets_agree(got, ref.rows[b], tau)
        assert ok, f"block row {b}: {why}; gpu {got} oracle {ref.rows[b]['kept']}"
        excused += bool(why)
    return excused
