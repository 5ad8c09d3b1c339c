"""Seeded synthetic workloads for the MapFlow hot path.

The shapes follow the model pairs the pages use (an 8B->3B pair with 32 sender heads and a
24-query / 8-KV-head receiver, a 14B->8B pair with 40 sender heads and a 32 / 8 receiver) and
the synthetic "planted key" recipe below.  Nothing here computes any step of the method; it
only draws random numbers and lays them out.

Recipe (one layer of one model pair; every draw is seeded with
``SeedSequence([seed, layer, tensor_id])`` so each tensor is reproducible on its own):

* ``z ~ N(0, I)`` independently for every (tensor, head, token).
* ``u_h`` is a random unit vector per sender head and layer (shared by Q and K).
* hot set: ``round(hot_frac * n)`` distinct positions drawn from ``[1, n)`` plus token 0, shared
  by all heads of the layer and redrawn per sequence.
* ``Q_s[h, t] = z + a * u_h`` at every token; ``K_s[h, t] = z + a * u_h`` at hot tokens and
  ``z`` elsewhere, with ``a = 0.75 * sqrt(d)``.
* ``W`` (receiver x sender head mixing weights): each row ~ Dirichlet(0.5, ..., 0.5).
* ``V_r ~ N(0, 1)``, layout ``[T, H_kv, d]``.
* bf16 workloads round Q, K and V to bf16 (round to nearest even); fp32 workloads keep fp32.
* varlen lengths are integers uniform on ``len_range`` (inclusive); pages are a seeded
  permutation of a pool that holds exactly the pages the sequences need.
* the densely recomputed receiver layers get plain ``N(0, 1)`` Q, K and V.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_TENSOR_IDS = {
    "q_s": 0, "k_s": 1, "u": 2, "hot": 3, "w": 4, "v_r": 5, "lens": 6, "pages": 7,
    "q_dense": 8, "k_dense": 9, "v_dense": 10,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    H_s: int
    H_r: int
    H_kv: int
    d: int
    B: int
    tau: float | None        # None: tuned per seed to a target kept-block density
    dtype: str               # "f32" or "bf16" for Q_s, K_s, V_r
    hot_frac: float
    seq_len: int | None = None
    n_seq: int = 1
    len_range: tuple[int, int] | None = None
    n_send_layers: int = 1
    n_recv_layers: int = 1
    R: int = 0               # receiver layers recomputed with dense causal attention
    paged: bool = False
    page_size: int = 16
    target_density: float | None = None


WORKLOADS = {
    "tiny": Workload(
        "tiny", "single layer, fp32: L=256, 4 sender heads -> 2 receiver heads, d=64, B=32",
        H_s=4, H_r=2, H_kv=2, d=64, B=32, tau=0.9, dtype="f32", hot_frac=0.01, seq_len=256),
    "pair_8b3b_8k": Workload(
        "pair_8b3b_8k", "8B->3B-class pair, one layer: L=8192, 32 -> 24q/8kv, d=128, B=64",
        H_s=32, H_r=24, H_kv=8, d=128, B=64, tau=0.95, dtype="bf16", hot_frac=0.01,
        seq_len=8192),
    "full_8b3b_32k": Workload(
        "full_8b3b_32k",
        "8B->3B full depth: L=32768, sender 36 layers x 32 heads, receiver 28 layers "
        "x 24q/8kv, d=128, B=64, first 2 receiver layers recomputed",
        H_s=32, H_r=24, H_kv=8, d=128, B=64, tau=0.95, dtype="bf16", hot_frac=0.01,
        seq_len=32768, n_send_layers=36, n_recv_layers=28, R=2),
    "varlen_14b8b": Workload(
        "varlen_14b8b",
        "14B->8B varlen packed batch: 16 sequences, lengths U[1024,16384], 40 -> 32q/8kv, "
        "d=128, B=64, V in 16-token pages",
        H_s=40, H_r=32, H_kv=8, d=128, B=64, tau=0.95, dtype="bf16", hot_frac=0.01,
        n_seq=16, len_range=(1024, 16384), paged=True, page_size=16),
    "long_131k": Workload(
        "long_131k",
        "long context: L=131072, 32 -> 24q/8kv, d=128, B=64, hot set 0.2%, tau tuned "
        "per seed to ~5% kept-block density",
        H_s=32, H_r=24, H_kv=8, d=128, B=64, tau=None, dtype="bf16", hot_frac=0.002,
        seq_len=131072, target_density=0.05),
}


def rng_for(seed: int, layer: int, tensor: str) -> np.random.Generator:
    """Independent numpy generator for one (seed, layer, tensor) triple."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(layer), _TENSOR_IDS[tensor]]))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_input_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(bf16_bits_from_f32(x))
    return x


def make_lengths(wl: Workload, seed: int, override: list[int] | None = None) -> list[int]:
    if override is not None:
        return [int(n) for n in override]
    if wl.len_range is None:
        return [int(wl.seq_len)] * wl.n_seq
    lo, hi = wl.len_range
    return [int(n) for n in rng_for(seed, 0, "lens").integers(lo, hi + 1, size=wl.n_seq)]


def cu_seqlens_of(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _unit_vectors(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _hot_positions(rng: np.random.Generator, n: int, frac: float) -> np.ndarray:
    n_hot = min(int(round(frac * n)), max(n - 1, 0))
    hot = rng.choice(np.arange(1, n), size=n_hot, replace=False) if n_hot > 0 else np.zeros(0, np.int64)
    return np.sort(np.concatenate([[0], hot])).astype(np.int64)


def make_layer_inputs(wl: Workload, seed: int, layer: int = 0, lengths: list[int] | None = None,
                      H_s: int | None = None, H_r: int | None = None, H_kv: int | None = None,
                      d: int | None = None) -> dict:
    """One sender layer (Q_s, K_s) and its mapped receiver layer (W, V_r) as numpy arrays.

    Q_s, K_s: float32 [H_s, T, d]; W: float32 [H_r, H_s]; V_r: float32 [T, H_kv, d].  For bf16
    workloads the float32 arrays hold bf16-representable values.  The head counts and d can be
    overridden to build smaller test cases with the same recipe.
    """
    H_s = H_s or wl.H_s
    H_r = H_r or wl.H_r
    H_kv = H_kv or wl.H_kv
    d = d or wl.d
    lengths = make_lengths(wl, seed, lengths)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    a = 0.75 * math.sqrt(d)
    u = _unit_vectors(rng_for(seed, layer, "u"), H_s, d).astype(np.float32)          # [H_s, d]
    q = rng_for(seed, layer, "q_s").standard_normal((H_s, T, d), dtype=np.float32)
    k = rng_for(seed, layer, "k_s").standard_normal((H_s, T, d), dtype=np.float32)
    q += np.float32(a) * u[:, None, :]
    hot_rng = rng_for(seed, layer, "hot")
    hot_tokens = []
    for s, n in enumerate(lengths):
        pos = _hot_positions(hot_rng, n, wl.hot_frac) + cu[s]
        hot_tokens.append(pos)
    hot_tokens = np.concatenate(hot_tokens) if hot_tokens else np.zeros(0, np.int64)
    k[:, hot_tokens, :] += np.float32(a) * u[:, None, :]
    w = rng_for(seed, layer, "w").dirichlet(np.full(H_s, 0.5), size=H_r).astype(np.float32)
    v = rng_for(seed, layer, "v_r").standard_normal((T, H_kv, d), dtype=np.float32)
    group = max(H_r // H_kv, 1)
    return {
        "q_s": _to_input_dtype(q, wl.dtype),
        "k_s": _to_input_dtype(k, wl.dtype),
        "w": w,
        "v_r": _to_input_dtype(v, wl.dtype),
        "cu_seqlens": cu,
        "lengths": lengths,
        "hot_tokens": hot_tokens,
        "kv_head_map": np.array([min(g // group, H_kv - 1) for g in range(H_r)], dtype=np.int32),
        "T": T, "H_s": H_s, "H_r": H_r, "H_kv": H_kv, "d": d, "B": wl.B, "dtype": wl.dtype,
    }


def make_dense_inputs(wl: Workload, seed: int, layer: int, lengths: list[int] | None = None,
                      H_q: int | None = None, H_kv: int | None = None, d: int | None = None) -> dict:
    """Plain N(0,1) Q [T, H_q, d], K and V [T, H_kv, d] for a densely recomputed receiver layer."""
    H_q = H_q or wl.H_r
    H_kv = H_kv or wl.H_kv
    d = d or wl.d
    lengths = make_lengths(wl, seed, lengths)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    q = rng_for(seed, layer, "q_dense").standard_normal((T, H_q, d), dtype=np.float32)
    k = rng_for(seed, layer, "k_dense").standard_normal((T, H_kv, d), dtype=np.float32)
    v = rng_for(seed, layer, "v_dense").standard_normal((T, H_kv, d), dtype=np.float32)
    return {"q": _to_input_dtype(q, wl.dtype), "k": _to_input_dtype(k, wl.dtype),
            "v": _to_input_dtype(v, wl.dtype), "cu_seqlens": cu, "lengths": lengths, "T": T}


def make_page_table(lengths, page_size: int, seed: int, layer: int = 0):
    """Shuffled page table: ``table[s, p]`` is the physical page of logical page p of sequence s.

    The pool holds exactly ``sum(ceil(n_s / page_size))`` pages; unused table entries are -1.
    """
    n_pages_seq = [(n + page_size - 1) // page_size for n in lengths]
    n_pages = int(sum(n_pages_seq))
    perm = rng_for(seed, layer, "pages").permutation(n_pages).astype(np.int32)
    width = max(n_pages_seq) if n_pages_seq else 0
    table = np.full((len(lengths), width), -1, dtype=np.int32)
    off = 0
    for s, np_s in enumerate(n_pages_seq):
        table[s, :np_s] = perm[off:off + np_s]
        off += np_s
    return table, n_pages


def page_v(v: np.ndarray, lengths, table: np.ndarray, page_size: int, n_pages: int) -> np.ndarray:
    """Scatter contiguous V [T, H_kv, d] into a page pool [n_pages, page_size, H_kv, d]."""
    pool = np.zeros((n_pages, page_size) + v.shape[1:], dtype=v.dtype)
    tok = 0
    for s, n in enumerate(lengths):
        for p in range((n + page_size - 1) // page_size):
            t0 = p * page_size
            t1 = min(n, t0 + page_size)
            pool[table[s, p], : t1 - t0] = v[tok + t0: tok + t1]
        tok += n
    return pool


# ----------------------------------------------------------------------------------------------
# Device-side bulk generation (same recipe, torch's generator instead of numpy's).  Used for
# multi-gigabyte benchmark inputs; the numbers differ from the numpy path, the distributions and
# structure do not.
# ----------------------------------------------------------------------------------------------
def _torch_gen(seed: int, layer: int, tensor: str, device):
    import torch
    state = np.random.SeedSequence([int(seed), int(layer), _TENSOR_IDS[tensor]]).generate_state(2)
    g = torch.Generator(device=device)
    g.manual_seed(int(state[0]) << 32 | int(state[1]))
    return g


def make_sender_inputs_torch(wl: Workload, seed: int, layer: int, device, lengths=None) -> dict:
    """Q_s, K_s [H_s, T, d] (input dtype) of one sender layer on ``device``."""
    import torch
    lengths = make_lengths(wl, seed, lengths)
    cu = cu_seqlens_of(lengths)
    T, H_s, d = int(cu[-1]), wl.H_s, wl.d
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    a = 0.75 * math.sqrt(d)
    u = torch.randn((H_s, d), generator=_torch_gen(seed, layer, "u", device), device=device)
    u = u / u.norm(dim=1, keepdim=True)
    boost = (a * u)[:, None, :]
    q = torch.randn((H_s, T, d), generator=_torch_gen(seed, layer, "q_s", device), device=device)
    q += boost
    q_out = q.to(dt)
    del q
    k = torch.randn((H_s, T, d), generator=_torch_gen(seed, layer, "k_s", device), device=device)
    g_hot = _torch_gen(seed, layer, "hot", device)
    hot = []
    for s, n in enumerate(lengths):
        n_hot = min(int(round(wl.hot_frac * n)), max(n - 1, 0))
        pos = torch.randperm(max(n - 1, 0), generator=g_hot, device=device)[:n_hot] + 1
        hot.append(torch.cat([torch.zeros(1, dtype=pos.dtype, device=device), pos]) + int(cu[s]))
    hot = torch.cat(hot)
    k[:, hot, :] += boost
    k_out = k.to(dt)
    del k
    return {"q_s": q_out, "k_s": k_out, "cu_seqlens": cu, "lengths": lengths, "T": T}


def make_receiver_inputs_torch(wl: Workload, seed: int, layer: int, device, lengths=None) -> dict:
    """W [H_r, H_s] fp32 and V_r [T, H_kv, d] (input dtype) of one mapped receiver layer."""
    import torch
    lengths = make_lengths(wl, seed, lengths)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    v = torch.randn((T, wl.H_kv, wl.d), generator=_torch_gen(seed, layer, "v_r", device), device=device).to(dt)
    w = torch.from_numpy(rng_for(seed, layer, "w").dirichlet(np.full(wl.H_s, 0.5), size=wl.H_r)
                         .astype(np.float32)).to(device)
    group = max(wl.H_r // wl.H_kv, 1)
    return {"w": w, "v_r": v, "cu_seqlens": cu, "lengths": lengths, "T": T,
            "kv_head_map": [min(g // group, wl.H_kv - 1) for g in range(wl.H_r)]}


def make_layer_inputs_torch(wl: Workload, seed: int, layer: int, device, lengths=None) -> dict:
    """Q_s, K_s [H_s, T, d], V_r [T, H_kv, d] (input dtype) and W [H_r, H_s] fp32 on ``device``:
    one sender layer and its receiver layer drawn with the same layer index."""
    out = make_sender_inputs_torch(wl, seed, layer, device, lengths)
    out.update(make_receiver_inputs_torch(wl, seed, layer, device, lengths))
    return out


def make_dense_inputs_torch(wl: Workload, seed: int, layer: int, device, lengths=None) -> dict:
    """Plain N(0,1) Q [T, H_r, d], K and V [T, H_kv, d] for a recomputed receiver layer."""
    import torch
    lengths = make_lengths(wl, seed, lengths)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = {}
    for name, H in [("q", wl.H_r), ("k", wl.H_kv), ("v", wl.H_kv)]:
        out[name] = torch.randn((T, H, wl.d), generator=_torch_gen(seed, layer, name + "_dense", device),
                                device=device).to(dt)
    group = max(wl.H_r // wl.H_kv, 1)
    out.update(cu_seqlens=cu, lengths=lengths, T=T,
               kv_head_map=[min(g // group, wl.H_kv - 1) for g in range(wl.H_r)])
    return out
