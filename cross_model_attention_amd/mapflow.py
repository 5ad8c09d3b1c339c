"""Python binding of libmapflow with the C ABI's names.

Argument marshalling only: every step of compress / retrieve / dense attention runs in the HIP
kernels of libmapflow.so.  PyTorch provides device memory and streams; tensors are passed to the
library as raw device pointers.  Nothing here falls back to a CPU or PyTorch implementation: if
the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import MfBsr, MfVfrag, check, i32_array

_L = _lib.load()


def version() -> str:
    return _L.mf_version().decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.MF_BF16
    if t.dtype == torch.float32:
        return _lib.MF_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _cu(cu_seqlens, T: int):
    if cu_seqlens is None:
        cu = [0, T]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return i32_array(cu), len(cu) - 1, cu


def _torch_allocator(device: int):
    """PyTorch's caching allocator as the library's device memory: every buffer the library owns
    (stores, prepared V, scratch) is taken from and returned to torch's pool."""

    def alloc(nbytes, stream):
        try:
            return torch.cuda.caching_allocator_alloc(int(nbytes), device, int(stream or 0))
        except torch.OutOfMemoryError:
            return None

    def free(ptr, nbytes, stream):
        torch.cuda.caching_allocator_delete(int(ptr))

    return alloc, free


class Context:
    """A libmapflow context on one device (owns scratch memory).

    ``allocator``: ``"torch"`` (the default: PyTorch's caching allocator provides all device
    memory), ``"hip"`` (hipMalloc / hipFree inside the library), or a pair ``(alloc, free)`` of
    callables ``alloc(nbytes, stream) -> device pointer or None`` and ``free(ptr, nbytes, stream)``.
    """

    _defaults: dict = {}

    def __init__(self, device: int = 0, allocator="torch"):
        if allocator == "hip":
            fns = None
        elif allocator == "torch":
            fns = _torch_allocator(int(device))
        else:
            fns = tuple(allocator)
        if fns is None:
            a, f = ctypes.cast(None, _lib.ALLOC_FN), ctypes.cast(None, _lib.FREE_FN)
        else:
            py_alloc, py_free = fns

            def _a(nbytes, stream, user):
                try:
                    p = py_alloc(nbytes, stream)
                    return int(p) if p else None
                except Exception:              # an exception must not unwind through C
                    return None

            def _f(ptr, nbytes, stream, user):
                try:
                    py_free(ptr, nbytes, stream)
                except Exception as e:         # noqa: BLE001 - reported, never propagated into C
                    print(f"libmapflow free callback failed: {e!r}", flush=True)

            a, f = _lib.ALLOC_FN(_a), _lib.FREE_FN(_f)
        self._callbacks = (a, f)               # must outlive every store and prepared V
        h = ctypes.c_void_p()
        check(_L.mf_create(int(device), a, f, None, ctypes.byref(h)))
        self.handle = h
        self.device = device

    @classmethod
    def default(cls, device: int | None = None) -> "Context":
        if device is None:
            device = torch.cuda.current_device()
        if device not in cls._defaults:
            cls._defaults[device] = Context(device)
        return cls._defaults[device]

    def close(self):
        if self.handle:
            _L.mf_destroy(self.handle)
            self.handle = None


def _ctx(ctx):
    return ctx if ctx is not None else Context.default()


# ----------------------------------------------------------------------------------------------
# block store layout helpers (host-side data movement)
# ----------------------------------------------------------------------------------------------
def probs_store_to_canonical(bits: np.ndarray, H_s: int) -> np.ndarray:
    """[nnzb, HG, B, B, 8] bf16 bits -> float64 [nnzb, H_s, B, B]."""
    f = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    n, HG, B, _, _ = f.shape
    return f.transpose(0, 1, 4, 2, 3).reshape(n, HG * 8, B, B)[:, :H_s].astype(np.float64)


def probs_canonical_to_store(probs: np.ndarray, H_s: int) -> np.ndarray:
    """float [nnzb, H_s, B, B] holding bf16 values -> uint16 bits [nnzb, HG, B, B, 8]."""
    n, H, B, _ = probs.shape
    HG = (H_s + 7) // 8
    full = np.zeros((n, HG * 8, B, B), dtype=np.float32)
    full[:, :H] = probs
    bits = (full.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if not np.array_equal((bits.astype(np.uint32) << np.uint32(16)).view(np.float32), full):
        raise ValueError("probs must hold bf16-representable values")
    return np.ascontiguousarray(bits.reshape(n, HG, 8, B, B).transpose(0, 1, 3, 4, 2))


class BlockStore:
    """An mf_bsr owned by the library (freed with the object)."""

    def __init__(self, ctx: Context, raw: MfBsr, cu: list[int]):
        self.ctx = ctx
        self.raw = raw
        self.cu_seqlens = cu

    @classmethod
    def create(cls, H_s: int, B: int, cu_seqlens, capacity: int = -1, ctx=None, row_begin=None) -> "BlockStore":
        """mf_bsr_create, or mf_bsr_create_range when ``row_begin`` (first block row per sequence)
        is given."""
        ctx = _ctx(ctx)
        cu_arr, n_seq, cu = _cu(cu_seqlens, 0)
        raw = MfBsr()
        if row_begin is None:
            check(_L.mf_bsr_create(ctx.handle, int(H_s), int(B), cu_arr, n_seq, int(capacity), ctypes.byref(raw)))
        else:
            if len(row_begin) != n_seq:
                raise ValueError("row_begin needs one entry per sequence")
            check(_L.mf_bsr_create_range(ctx.handle, int(H_s), int(B), cu_arr, n_seq, i32_array(row_begin),
                                         int(capacity), ctypes.byref(raw)))
        return cls(ctx, raw, cu)

    def __getattr__(self, name):
        raw = self.__dict__.get("raw")
        if raw is not None and name in dict(MfBsr._fields_):
            return getattr(raw, name)
        raise AttributeError(name)

    def sync(self, stream=None) -> int:
        check(_L.mf_bsr_sync(self.ctx.handle, ctypes.byref(self.raw), _stream(stream)))
        return self.raw.nnzb

    def to_host(self) -> dict:
        r = self.raw
        ptr = np.zeros(r.n_brow + 1, np.int32)
        check(_L.mf_bsr_download(self.ctx.handle, ctypes.byref(r), ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 None, None, None))
        n = int(r.nnzb)
        HG = (r.H_s + 7) // 8
        idx = np.zeros(max(n, 1), np.int32)
        bits = np.zeros((max(n, 1), HG, r.B, r.B, 8), np.uint16)
        rkm = np.zeros((r.H_s, max(r.T, 1)), np.float32)
        check(_L.mf_bsr_download(self.ctx.handle, ctypes.byref(r),
                                 ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                 rkm.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        return {"block_ptr": ptr, "block_idx": idx[:n], "probs_bits": bits[:n],
                "probs": probs_store_to_canonical(bits[:n], r.H_s), "row_kept_mass": rkm[:, : r.T],
                "nnzb": n}

    def meta_to_host(self) -> dict:
        """block_ptr and row_kept_mass only (no probabilities)."""
        r = self.raw
        ptr = np.zeros(r.n_brow + 1, np.int32)
        rkm = np.zeros((r.H_s, max(r.T, 1)), np.float32)
        check(_L.mf_bsr_download(self.ctx.handle, ctypes.byref(r),
                                 ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, None,
                                 rkm.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        return {"block_ptr": ptr, "row_kept_mass": rkm[:, : r.T], "nnzb": int(r.nnzb)}

    def blocks_to_host(self, first: int, count: int, probs: bool = True) -> dict:
        """Kept blocks [first, first + count): columns and (optionally) canonical probs
        [count, H_s, B, B]."""
        r = self.raw
        n = max(int(count), 1)
        idx = np.zeros(n, np.int32)
        bits = np.zeros((n, (r.H_s + 7) // 8, r.B, r.B, 8), np.uint16) if probs else None
        check(_L.mf_bsr_download_blocks(
            self.ctx.handle, ctypes.byref(r), int(first), int(count),
            idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)) if probs else None))
        out = {"block_idx": idx[:count]}
        if probs:
            out["probs"] = probs_store_to_canonical(bits[:count], r.H_s)
        return out

    def upload(self, block_ptr, block_idx, probs, row_kept_mass) -> None:
        """Fill from host arrays; ``probs`` canonical [nnzb, H_s, B, B] with bf16 values."""
        r = self.raw
        ptr = np.ascontiguousarray(block_ptr, dtype=np.int32)
        idx = np.ascontiguousarray(block_idx, dtype=np.int32)
        bits = probs_canonical_to_store(np.asarray(probs, dtype=np.float32), r.H_s)
        rkm = np.ascontiguousarray(row_kept_mass, dtype=np.float32)
        check(_L.mf_bsr_upload(self.ctx.handle, ctypes.byref(r),
                               ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                               rkm.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))

    def free(self):
        if self.__dict__.get("borrowed_from") is not None:
            return                                   # a prefix-cache entry: the cache owns it
        if self.__dict__.get("raw") is not None and self.raw._owner:
            _L.mf_bsr_free(self.ctx.handle, ctypes.byref(self.raw))

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _tokens(tokens):
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    return t, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def prefix_hashes(tokens, B: int) -> np.ndarray:
    """mf_prefix_hashes: chained hash of every full B-token block of ``tokens`` (host only)."""
    t, tp = _tokens(tokens)
    out = np.zeros(len(t) // int(B), dtype=np.uint64)
    check(_L.mf_prefix_hashes(tp, len(t), int(B), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))))
    return out


class PrefixCache:
    """mf_cache: compressed block rows of token prefixes, per layer, found by prefix hash."""

    def __init__(self, budget_bytes: int, ctx=None):
        self.ctx = _ctx(ctx)
        h = ctypes.c_void_p()
        check(_L.mf_cache_create(self.ctx.handle, int(budget_bytes), ctypes.byref(h)))
        self.handle = h

    def insert(self, layer: int, tokens, parts, rows: int, stream=None) -> None:
        """Cache block rows 0..rows-1 of ``tokens``, taking each row from the first of ``parts``
        (single-sequence stores, e.g. a looked-up prefix and a row-range store) that compressed it."""
        t, tp = _tokens(tokens)
        arr = (MfBsr * len(parts))(*[p.raw for p in parts])
        check(_L.mf_cache_insert(self.handle, int(layer), tp, len(t), len(parts), arr, int(rows), _stream(stream)))

    def lookup(self, layer: int, tokens, B: int):
        """Longest cached prefix: (rows, store view of rows 0..rows-1) or (0, None).  The view
        stays valid until an insert evicts it or the cache is closed."""
        t, tp = _tokens(tokens)
        rows = ctypes.c_int32(0)
        raw = MfBsr()
        check(_L.mf_cache_lookup(self.handle, int(layer), tp, len(t), int(B), ctypes.byref(rows), ctypes.byref(raw)))
        if rows.value == 0:
            return 0, None
        view = BlockStore(self.ctx, raw, [0, rows.value * int(B)])
        view.borrowed_from = self
        return rows.value, view

    def info(self):
        n, used = ctypes.c_int64(0), ctypes.c_int64(0)
        check(_L.mf_cache_info(self.handle, ctypes.byref(n), ctypes.byref(used)))
        return n.value, used.value

    def close(self):
        if self.__dict__.get("handle"):
            _L.mf_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PreparedV:
    """An mf_vfrag (receiver V in MFMA operand layout), owned by the library."""

    def __init__(self, ctx: Context, raw: MfVfrag):
        self.ctx = ctx
        self.raw = raw

    def free(self):
        if self.__dict__.get("raw") is not None and self.raw._owner:
            _L.mf_vfrag_free(self.ctx.handle, ctypes.byref(self.raw))

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ----------------------------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------------------------
def layer_map_uniform(n_recv: int, n_send: int, R: int) -> list[int]:
    """mf_layer_map_uniform: -1 for the first R layers, then round(l (n_send-1) / (n_recv-1))."""
    out = (ctypes.c_int32 * n_recv)()
    check(_L.mf_layer_map_uniform(int(n_recv), int(n_send), int(R), out))
    return list(out)


def map_layers(pi, n_send: int, R: int, ctx=None) -> None:
    """mf_map_layers: install the layer map ``pi`` (one entry per receiver layer) on the context."""
    ctx = _ctx(ctx)
    check(_L.mf_map_layers(ctx.handle, i32_array(pi), len(pi), int(n_send), int(R)))


def check_layer_map(pi, n_recv: int, n_send: int, R: int) -> None:
    check(_L.mf_check_layer_map(i32_array(pi), int(n_recv), int(n_send), int(R)))


def _check_qk(Q, K):
    if Q.dim() != 3 or K.shape != Q.shape:
        raise ValueError(f"Q and K must both be [H_s, T, d] (got {tuple(Q.shape)}, {tuple(K.shape)})")
    if Q.dtype != K.dtype:
        raise TypeError("Q and K must have the same dtype")


def compress(Q: torch.Tensor, K: torch.Tensor, tau: float, B: int, cu_seqlens=None, ctx=None,
             stream=None) -> BlockStore:
    """mf_compress: exactly sized block store of one sender layer (Q, K: [H_s, T, d])."""
    ctx = _ctx(ctx)
    _check_qk(Q, K)
    H_s, T, d = Q.shape
    cu_arr, n_seq, cu = _cu(cu_seqlens, T)
    raw = MfBsr()
    check(_L.mf_compress(ctx.handle, _dev(Q, "Q"), _dev(K, "K"), _dtype(Q), int(H_s), int(d),
                         cu_arr, n_seq, float(tau), int(B), _stream(stream), ctypes.byref(raw)))
    return BlockStore(ctx, raw, cu)


def compress_into(store: BlockStore, Q: torch.Tensor, K: torch.Tensor, tau: float, stream=None,
                  per_head_select: bool = False, per_head_norm: bool = False) -> None:
    """mf_compress_into (or mf_compress_into_ex with the variant options): asynchronous compress
    into a preallocated store."""
    _check_qk(Q, K)
    if Q.shape[0] != store.raw.H_s or Q.shape[1] != store.raw.T:
        raise ValueError("Q/K shape does not match the store's geometry")
    opts = (1 if per_head_select else 0) | (2 if per_head_norm else 0)
    if opts:
        check(_L.mf_compress_into_ex(store.ctx.handle, _dev(Q, "Q"), _dev(K, "K"), _dtype(Q), int(Q.shape[2]),
                                     float(tau), opts, ctypes.byref(store.raw), _stream(stream)))
    else:
        check(_L.mf_compress_into(store.ctx.handle, _dev(Q, "Q"), _dev(K, "K"), _dtype(Q), int(Q.shape[2]),
                                  float(tau), ctypes.byref(store.raw), _stream(stream)))


def compress_prefill_into(store: BlockStore, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, tau: float,
                          out=None, stream=None) -> torch.Tensor:
    """mf_compress_prefill_into: the sender's causal attention O [T, H_s, d] fp32 and the store,
    from one pass over the scores.  V: [T, H_s, d], dtype as Q."""
    _check_qk(Q, K)
    H_s, T, d = Q.shape
    if H_s != store.raw.H_s or T != store.raw.T:
        raise ValueError("Q/K shape does not match the store's geometry")
    if V.shape != (T, H_s, d) or V.dtype != Q.dtype:
        raise ValueError("V must be [T, H_s, d] with Q's dtype")
    out = _out(out, T, H_s, d, Q)
    check(_L.mf_compress_prefill_into(store.ctx.handle, _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dtype(Q), int(d),
                                      float(tau), ctypes.byref(store.raw), _dev(out, "out"), _stream(stream)))
    return out


def _paged(page_table, page_size):
    if page_table is None:
        return None, 0, 0
    return _dev(page_table, "page_table"), int(page_size), int(page_table.shape[1])


def v_prepare(V: torch.Tensor, B: int, cu_seqlens=None, page_table=None, page_size: int = 16,
              out: PreparedV | None = None, ctx=None, stream=None) -> PreparedV:
    """mf_v_prepare.  V: [T, H_kv, d] contiguous, or a page pool [n_pages, page_size, H_kv, d].
    With ``out`` (same geometry) the preparation is redone in place without allocating."""
    ctx = out.ctx if out is not None else _ctx(ctx)
    H_kv, d = int(V.shape[-2]), int(V.shape[-1])
    if page_table is None and cu_seqlens is None:
        cu_seqlens = [0, int(V.shape[0])]
    if cu_seqlens is None:
        raise ValueError("paged V needs cu_seqlens")
    cu_arr, n_seq, _ = _cu(cu_seqlens, 0)
    pt, ps, pps = _paged(page_table, page_size)
    raw = out.raw if out is not None else MfVfrag()
    check(_L.mf_v_prepare(ctx.handle, cu_arr, n_seq, int(B), _dev(V, "V"), _dtype(V), H_kv, d, pt, ps,
                          pps, ctypes.byref(raw), _stream(stream)))
    return out if out is not None else PreparedV(ctx, raw)


def _out(out, T, H, d, like):
    if out is None:
        return torch.empty((T, H, d), dtype=torch.float32, device=like.device)
    if out.shape != (T, H, d) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [T, H, d]")
    return out


def retrieve_prepared(store: BlockStore, W: torch.Tensor, pv: PreparedV, kv_head_map, out=None,
                      stream=None) -> torch.Tensor:
    """mf_retrieve_prepared: O [T, H_r, d] fp32 from the store, W [H_r, H_s] fp32 and prepared V."""
    H_r = int(W.shape[0])
    if W.dtype != torch.float32 or W.shape[1] != store.raw.H_s:
        raise ValueError("W must be float32 [H_r, H_s]")
    out = _out(out, store.raw.T, H_r, pv.raw.d, W)
    check(_L.mf_retrieve_prepared(store.ctx.handle, ctypes.byref(store.raw), _dev(W, "W"), H_r,
                                  ctypes.byref(pv.raw), i32_array(kv_head_map), _dev(out, "out"),
                                  _stream(stream)))
    return out


def retrieve_multi(store: BlockStore, receivers, outs=None, stream=None) -> list[torch.Tensor]:
    """mf_retrieve_multi: one launch for several receivers of the same store.

    ``receivers`` is a sequence of ``(W, prepared_v, kv_head_map)``; returns one O [T, H_r, d] fp32
    per receiver (or fills ``outs``)."""
    receivers = list(receivers)
    n = len(receivers)
    if outs is not None and len(outs) != n:
        raise ValueError("outs must have one tensor per receiver")
    Ws, Hs, vfs, maps, Os, tensors = [], [], [], [], [], []
    for r, (W, pv, kvmap) in enumerate(receivers):
        if W.dtype != torch.float32 or W.dim() != 2 or W.shape[1] != store.raw.H_s:
            raise ValueError(f"W of receiver {r} must be float32 [H_r, H_s]")
        H_r = int(W.shape[0])
        out = _out(None if outs is None else outs[r], store.raw.T, H_r, pv.raw.d, W)
        m = i32_array(kvmap)
        tensors.append(out)
        Ws.append(_dev(W, "W"))
        Hs.append(H_r)
        vfs.append(ctypes.pointer(pv.raw))
        maps.append(ctypes.cast(m, _lib._P_I32))
        Os.append(_dev(out, "out"))
    W_arr = (ctypes.c_void_p * n)(*Ws)
    H_arr = (ctypes.c_int32 * n)(*Hs)
    vf_arr = (ctypes.POINTER(MfVfrag) * n)(*vfs)
    map_arr = (_lib._P_I32 * n)(*maps)
    O_arr = (ctypes.c_void_p * n)(*Os)
    check(_L.mf_retrieve_multi(store.ctx.handle, ctypes.byref(store.raw), n, W_arr, H_arr, vf_arr,
                               map_arr, O_arr, _stream(stream)))
    return tensors


def retrieve_layers(stores, Ws, pv: PreparedV, kv_head_map, out=None, stream=None) -> torch.Tensor:
    """mf_retrieve_layers: one receiver layer from several sender layers' stores; Ws[l] is fp32
    [H_r, stores[l].H_s]."""
    stores, Ws = list(stores), list(Ws)
    if len(stores) != len(Ws) or not stores:
        raise ValueError("one W per store")
    H_r = int(Ws[0].shape[0])
    for st, W in zip(stores, Ws):
        if W.dtype != torch.float32 or W.dim() != 2 or W.shape != (H_r, st.raw.H_s):
            raise ValueError("each W must be float32 [H_r, H_s of its store]")
    out = _out(out, stores[0].raw.T, H_r, pv.raw.d, Ws[0])
    arr = (MfBsr * len(stores))(*[st.raw for st in stores])
    w_arr = (ctypes.c_void_p * len(Ws))(*[_dev(W, "W") for W in Ws])
    check(_L.mf_retrieve_layers(stores[0].ctx.handle, len(stores), arr, w_arr, H_r, ctypes.byref(pv.raw),
                                i32_array(kv_head_map), _dev(out, "out"), _stream(stream)))
    return out


def retrieve(store: BlockStore, W: torch.Tensor, V: torch.Tensor, kv_head_map, page_table=None,
             page_size: int = 16, out=None, stream=None) -> torch.Tensor:
    """mf_retrieve: V preparation into context scratch + the fused retrieve kernel."""
    H_r = int(W.shape[0])
    if W.dtype != torch.float32 or W.shape[1] != store.raw.H_s:
        raise ValueError("W must be float32 [H_r, H_s]")
    H_kv, d = int(V.shape[-2]), int(V.shape[-1])
    out = _out(out, store.raw.T, H_r, d, W)
    pt, ps, pps = _paged(page_table, page_size)
    check(_L.mf_retrieve(store.ctx.handle, ctypes.byref(store.raw), _dev(W, "W"), H_r, _dev(V, "V"),
                         _dtype(V), H_kv, d, pt, ps, pps, i32_array(kv_head_map), _dev(out, "out"),
                         _stream(stream)))
    return out


def retrieve_noalloc(store: BlockStore, W: torch.Tensor, V: torch.Tensor, kv_head_map, page_table=None,
                     page_size: int = 16, out=None, stream=None) -> torch.Tensor:
    """mf_retrieve_noalloc: mf_retrieve with the prepared V in the library's fixed device array (no
    device allocation inside the call).  ``out`` should be given by callers that must not allocate."""
    H_r = int(W.shape[0])
    if W.dtype != torch.float32 or W.shape[1] != store.raw.H_s:
        raise ValueError("W must be float32 [H_r, H_s]")
    H_kv, d = int(V.shape[-2]), int(V.shape[-1])
    out = _out(out, store.raw.T, H_r, d, W)
    pt, ps, pps = _paged(page_table, page_size)
    check(_L.mf_retrieve_noalloc(store.ctx.handle, ctypes.byref(store.raw), _dev(W, "W"), H_r, _dev(V, "V"),
                                 _dtype(V), H_kv, d, pt, ps, pps, i32_array(kv_head_map), _dev(out, "out"),
                                 _stream(stream)))
    return out


def dense_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv_head_map, cu_seqlens=None,
                    out=None, ctx=None, stream=None) -> torch.Tensor:
    """mf_dense_attention: causal softmax attention, Q [T, H_q, d], K/V [T, H_kv, d] -> fp32 O."""
    ctx = _ctx(ctx)
    T, H_q, d = Q.shape
    H_kv = int(K.shape[1])
    if K.shape != V.shape or K.shape[0] != T or K.shape[2] != d:
        raise ValueError("K and V must be [T, H_kv, d] matching Q")
    cu_arr, n_seq, _ = _cu(cu_seqlens, T)
    out = _out(out, T, H_q, d, Q)
    check(_L.mf_dense_attention(ctx.handle, _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dtype(Q), H_q,
                                H_kv, d, cu_arr, n_seq, i32_array(kv_head_map), _dev(out, "out"),
                                _stream(stream)))
    return out


def copy_probe(dst: torch.Tensor, src: torch.Tensor, ctx=None, stream=None) -> None:
    ctx = _ctx(ctx)
    nbytes = src.numel() * src.element_size()
    check(_L.mf_copy_probe(ctx.handle, _dev(dst, "dst"), _dev(src, "src"), nbytes, _stream(stream)))


def write_probe(dst: torch.Tensor, src: torch.Tensor | None = None, ctx=None, stream=None) -> None:
    """mf_write_probe: fill dst with coalesced non-temporal stores, reading one 16-byte record of
    src per five written when src is given (the gather's read : write mix)."""
    ctx = _ctx(ctx)
    nbytes = dst.numel() * dst.element_size()
    if src is not None and src.numel() * src.element_size() < nbytes // 5:
        raise ValueError("src needs bytes / 5")
    check(_L.mf_write_probe(ctx.handle, _dev(dst, "dst"), nbytes, None if src is None else _dev(src, "src"),
                            _stream(stream)))


def fill_probe(dst: torch.Tensor, value: int, ctx=None, stream=None) -> None:
    """mf_fill_probe: write the 32-bit value to every word of dst with plain stores in 256 KiB
    runs (the device's write ceiling)."""
    ctx = _ctx(ctx)
    nbytes = dst.numel() * dst.element_size()
    check(_L.mf_fill_probe(ctx.handle, _dev(dst, "dst"), nbytes, value & 0xFFFFFFFF, _stream(stream)))


def read_probe(src: torch.Tensor, sink: torch.Tensor, ctx=None, stream=None) -> None:
    """mf_read_probe: stream src through non-temporal loads (HBM read ceiling); sink is a device
    tensor of at least 4 bytes that the probe leaves untouched."""
    ctx = _ctx(ctx)
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink needs 4 bytes")
    check(_L.mf_read_probe(ctx.handle, _dev(src, "src"), nbytes, _dev(sink, "sink"), _stream(stream)))


def prefill_layers(slots, send, recv, kv_head_map, tau: float, isolate: bool = False, timing: bool = False,
                   ctx=None, stream_main=None, stream_prefetch=None) -> None:
    """mf_prefill_layers: one receiver prefill over every layer of the installed layer map.

    ``slots``: list of BlockStore (the ring); ``send``: per sender layer a (Q, K) pair of
    [H_s, T, d] tensors, or None for layers no receiver layer reuses; ``recv``: per receiver layer
    a dict with ``v`` and ``o`` [T, H, d] plus ``q``, ``k`` (recomputed layers) or ``w`` [H_r, H_s]
    (mapped layers).  Work goes on ``stream_main`` (default: the current stream) and
    ``stream_prefetch`` (required)."""
    ctx = _ctx(ctx)
    if stream_prefetch is None:
        raise ValueError("stream_prefetch is required")
    rl = (_lib.MfRecvLayer * len(recv))()
    v0 = None
    for i, r in enumerate(recv):
        def ptr(name):
            t = r.get(name)
            return None if t is None else _dev(t, f"recv[{i}].{name}")
        rl[i] = _lib.MfRecvLayer(ptr("q"), ptr("k"), ptr("v"), ptr("w"), ptr("o"))
        if v0 is None and r.get("v") is not None:
            v0, o0 = r["v"], r["o"]
    sl = (_lib.MfSendLayer * len(send))()
    for i, pair in enumerate(send):
        if pair is not None:
            sl[i] = _lib.MfSendLayer(_dev(pair[0], f"send[{i}].Q"), _dev(pair[1], f"send[{i}].K"))
    arr = (MfBsr * len(slots))(*[st.raw for st in slots])
    H_kv, d = int(v0.shape[-2]), int(v0.shape[-1])
    H_r = int(o0.shape[1])
    flags = (_lib.MF_PREFILL_ISOLATE if isolate else 0) | (_lib.MF_PREFILL_TIMING if timing else 0)
    check(_L.mf_prefill_layers(ctx.handle, rl, sl, _dtype(v0), H_r, H_kv, d, i32_array(kv_head_map), float(tau),
                               len(slots), arr, flags, _stream(stream_main), _stream(stream_prefetch)))
    for st, raw in zip(slots, arr):           # the library may update counts in the copies
        st.raw.nnzb = raw.nnzb


def prefill_timings(n_dense: int, n_map: int, ctx=None) -> dict:
    """mf_prefill_timings: per-stage milliseconds of the last timed prefill_layers call."""
    ctx = _ctx(ctx)
    out = {k: (ctypes.c_float * max(n, 1))() for k, n in
           (("dense", n_dense), ("compress", n_map), ("vprep", n_map), ("retrieve", n_map))}
    check(_L.mf_prefill_timings(ctx.handle, out["dense"], out["compress"], out["vprep"], out["retrieve"]))
    return {"dense": list(out["dense"])[:n_dense], "compress": list(out["compress"])[:n_map],
            "vprep": list(out["vprep"])[:n_map], "retrieve": list(out["retrieve"])[:n_map]}
