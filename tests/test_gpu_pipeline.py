"""GPU tests of the receiver-prefill pipeline (mf_prefill_layers) and of the caller's allocator.

The pipeline runs the dense recompute of the first R receiver layers on one stream while a second
stream compresses the sender layers of the first mapped layers into a ring of stores, then the
fused retrieve of every mapped layer, refilling each slot once its retrieve has finished
([MapFlow开源, section 2. 找得快的:基于前缀哈希的缓存管理]: later layers' blocks load in the
background while the first layers compute).  Checked here, on a reduced-depth version of the
8B->3B full-depth workload (8 sender layers, 6 receiver layers of which 2 recomputed, a 2-slot
ring, a ragged last block row):

* every output equals, bit for bit, a one-stream serial run of the same calls (compress of each
  mapped layer into its own store, V preparation, retrieve; dense attention), in both the
  isolated and the overlapped schedule, and again on a second call that reuses the ring;
* each mapped layer's selection matches the oracle's (tie rule) and its output matches the oracle
  run on the GPU's own stored blocks; each recomputed layer matches the oracle's dense attention;
* the stage timings are readable.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_out_close, check_selection, gpu_store_for_oracle, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mf():
    import cross_model_attention_amd as m
    return m


def _pipeline_case(L, n_send, n_recv, R, H_s, H_r, H_kv, d, seed):
    wl = synth.WORKLOADS["full_8b3b_32k"]
    pi = oracle.layer_map(n_recv, n_send, R)
    send, recv = [None] * n_send, []
    for j in sorted({p for p in pi if p >= 0}):
        x = synth.make_layer_inputs(wl, seed, layer=j, lengths=[L], H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
        send[j] = {"q": x["q_s"], "k": x["k_s"]}
    for l in range(n_recv):
        if pi[l] < 0:
            x = synth.make_dense_inputs(wl, seed, layer=l, lengths=[L], H_q=H_r, H_kv=H_kv, d=d)
            recv.append({"q": x["q"], "k": x["k"], "v": x["v"]})
        else:
            x = synth.make_layer_inputs(wl, seed, layer=100 + l, lengths=[L], H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
            recv.append({"w": x["w"], "v": x["v_r"]})
    kv = [g // (H_r // H_kv) for g in range(H_r)]
    return pi, send, recv, kv, float(np.float32(wl.tau)), wl.B


def _to_device(send, recv):
    dsend = [None if s is None else (to_dev(s["q"], "bf16"), to_dev(s["k"], "bf16")) for s in send]
    drecv = []
    for r in recv:
        e = {k: to_dev(v, torch.float32 if k == "w" else "bf16") for k, v in r.items()}
        drecv.append(e)
    return dsend, drecv


def _outs(recv, L, H_r, d):
    return [torch.full((L, H_r, d), float("nan"), device="cuda") for _ in recv]


@pytest.mark.parametrize("isolate", [True, False])
def test_prefill_pipeline_matches_serial_run_and_oracle(mf, isolate):
    L, n_send, n_recv, R = 1000, 8, 6, 2
    H_s, H_r, H_kv, d = 32, 24, 8, 128
    pi, send, recv, kv, tau, B = _pipeline_case(L, n_send, n_recv, R, H_s, H_r, H_kv, d, seed=21)
    say(f"case: prefill pipeline isolate={isolate} L={L} pi={pi} slots=2")
    dsend, drecv = _to_device(send, recv)
    cu = [0, L]
    mf.map_layers(pi, n_send, R)
    slots = [mf.BlockStore.create(H_s, B, cu) for _ in range(2)]
    s_main, s_pre = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for call in range(2):                               # the second call reuses the ring
        O = _outs(recv, L, H_r, d)
        for r, o in zip(drecv, O):
            r["o"] = o
        torch.cuda.current_stream().synchronize()
        mf.prefill_layers(slots, dsend, drecv, kv, tau, isolate=isolate, timing=True,
                          stream_main=s_main, stream_prefetch=s_pre)
        s_main.synchronize()
        outs.append(O)
        t = mf.prefill_timings(R, n_recv - R)
        assert all(v > 0 for k in t for v in t[k]), t
        say(f"  call {call}: retrieve ms {['%.3f' % v for v in t['retrieve']]}")
    # one-stream serial run of the same calls
    mapped = [l for l in range(n_recv) if pi[l] >= 0]
    serial, stores = {}, {}
    for l in range(n_recv):
        r = drecv[l]
        if pi[l] < 0:
            serial[l] = mf.dense_attention(r["q"], r["k"], r["v"], kv, cu_seqlens=cu)
        else:
            st = mf.BlockStore.create(H_s, B, cu)
            mf.compress_into(st, *dsend[pi[l]], tau)
            pv = mf.v_prepare(r["v"], B, cu)
            serial[l] = mf.retrieve_prepared(st, r["w"], pv, kv)
            stores[l] = st
    torch.cuda.synchronize()
    for call, O in enumerate(outs):
        for l in range(n_recv):
            assert torch.equal(O[l], serial[l]), f"call {call}: layer {l} differs from the serial run"
    # the ring holds the last two mapped layers' stores
    for i, l in enumerate(mapped[-2:]):
        m = len(mapped) - 2 + i
        a, b = slots[m % 2].to_host(), stores[l].to_host()
        for key in ["block_ptr", "block_idx", "probs_bits", "row_kept_mass"]:
            assert np.array_equal(a[key], b[key]), f"slot of layer {l}: {key}"
    # against the oracle
    for l in range(n_recv):
        got = outs[0][l].cpu().numpy()
        if pi[l] < 0:
            ref = oracle.dense_causal_attention(recv[l]["q"], recv[l]["k"], recv[l]["v"], np.array(cu), kv)
            assert_out_close(got, ref, f"layer {l} (dense)")
            continue
        host = stores[l].to_host()
        ref = oracle.compress(send[pi[l]]["q"], send[pi[l]]["k"], np.array(cu), tau, B)
        ex = check_selection(host, ref, tau, B)
        gs = gpu_store_for_oracle(host, cu, B, H_s)
        assert_out_close(got, oracle.retrieve(gs, recv[l]["w"], recv[l]["v"], kv),
                         f"layer {l} (sender layer {pi[l]}, {host['nnzb']} blocks, {ex} tie rows)")


def test_prefill_pipeline_rejects_bad_rings(mf):
    L, H_s, B = 300, 8, 64
    pi, send, recv, kv, tau, _ = _pipeline_case(L, 3, 3, 1, H_s, 8, 2, 64, seed=22)
    dsend, drecv = _to_device(send, recv)
    for r, o in zip(drecv, _outs(recv, L, 8, 64)):
        r["o"] = o
    mf.map_layers(pi, 3, 1)
    s2 = torch.cuda.Stream()
    small = mf.BlockStore.create(H_s, B, [0, L], capacity=3)
    with pytest.raises(mf.MapflowError, match="causal blocks"):
        mf.prefill_layers([small], dsend, drecv, kv, tau, stream_prefetch=s2)
    other = mf.BlockStore.create(H_s, B, [0, L - 1])
    full = mf.BlockStore.create(H_s, B, [0, L])
    with pytest.raises(mf.MapflowError, match="geometry"):
        mf.prefill_layers([full, other], dsend, drecv, kv, tau, stream_prefetch=s2)
    ranged = mf.BlockStore.create(H_s, B, [0, L], row_begin=[1])
    with pytest.raises(mf.MapflowError, match="row-range"):
        mf.prefill_layers([ranged], dsend, drecv, kv, tau, stream_prefetch=s2)
    drecv[0]["q"] = None                                 # a recomputed layer without queries
    with pytest.raises(mf.MapflowError, match="Q or K"):
        mf.prefill_layers([full], dsend, drecv, kv, tau, stream_prefetch=s2)
    torch.cuda.synchronize()


class _Budget:
    """A caller allocator over torch's caching allocator that refuses past a byte budget and
    records what is live."""

    def __init__(self, budget):
        self.budget = budget
        self.live = {}
        self.taken = self.given = self.refused = 0

    def alloc(self, nbytes, stream):
        if sum(self.live.values()) + nbytes > self.budget:
            self.refused += 1
            return None
        p = torch.cuda.caching_allocator_alloc(int(nbytes), 0, int(stream or 0))
        self.live[p] = nbytes
        self.taken += 1
        return p

    def free(self, ptr, nbytes, stream):
        assert self.live.pop(ptr) == nbytes, "freed with another size than allocated"
        torch.cuda.caching_allocator_delete(ptr)
        self.given += 1


class _FailNth(_Budget):
    """Refuses exactly the n-th allocation request (1-based) and grants every other."""

    def __init__(self, n):
        super().__init__(1 << 50)
        self.n, self.calls = n, 0

    def alloc(self, nbytes, stream):
        self.calls += 1
        if self.calls == self.n:
            self.refused += 1
            return None
        return super().alloc(nbytes, stream)


def _workflow(mf, ctx, x, tau, B):
    """Create, compress, prepare V, retrieve, fan out to two receivers: every allocating call."""
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    store = mf.BlockStore.create(x["H_s"], B, x["cu_seqlens"], ctx=ctx)
    objs = [store]
    mf.compress_into(store, Q, K, tau)
    pv = mf.v_prepare(V, B, x["cu_seqlens"], ctx=ctx)
    objs.append(pv)
    O = mf.retrieve_prepared(store, W, pv, x["kv_head_map"])
    outs = mf.retrieve_multi(store, [(W, pv, x["kv_head_map"]), (W, pv, x["kv_head_map"])])
    torch.cuda.synchronize()
    return objs, O, outs


@pytest.mark.parametrize("n", range(1, 16))
def test_each_allocation_failing_leaks_nothing(mf, n):
    """Refusing the n-th device allocation of a whole workflow (store, statistics and gather
    scratch, prepared V, retrieve tables) turns that call into MF_ERR_OOM, leaves every buffer of
    the context accounted for, and the same workflow succeeds afterwards with the same results as
    an unrestricted context."""
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 70, lengths=[300, 70], H_s=8, H_r=6, H_kv=2, d=64)
    tau = float(np.float32(wl.tau))
    say(f"case: the allocation number {n} of the workflow is refused")
    ref_ctx = mf.Context(0, allocator="hip")
    ref_objs, ref_O, ref_outs = _workflow(mf, ref_ctx, x, tau, wl.B)
    al = _FailNth(n)
    ctx = mf.Context(0, allocator=(al.alloc, al.free))
    objs = []
    try:
        objs, O, outs = _workflow(mf, ctx, x, tau, wl.B)
        failed = False
    except mf.MapflowError as e:
        assert "OOM" in str(e), str(e)
        failed = True
    assert failed == (al.refused == 1)
    if n == 15:                    # the largest n is past the workflow's last request: all covered
        assert not failed and al.calls < n, al.calls
    if not failed:
        assert torch.equal(O, ref_O) and all(torch.equal(a, b) for a, b in zip(outs, ref_outs))
    # with nothing refused any more the workflow runs on the same context and matches
    al.n = -1
    objs2, O2, outs2 = _workflow(mf, ctx, x, tau, wl.B)
    assert torch.equal(O2, ref_O) and all(torch.equal(a, b) for a, b in zip(outs2, ref_outs))
    for o in objs + objs2:
        o.free()
    ctx.close()
    assert al.live == {}, f"{len(al.live)} buffers still held"
    assert al.taken == al.given
    for o in ref_objs:
        o.free()
    ref_ctx.close()


def test_caller_allocator_provides_every_buffer_and_oom_leaks_nothing(mf):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    x = synth.make_layer_inputs(wl, 23, lengths=[600, 130], H_s=16, H_r=12, H_kv=4, d=128)
    tau = float(np.float32(wl.tau))
    say("case: caller allocator and out-of-memory")
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    W, V = to_dev(x["w"]), to_dev(x["v_r"], "bf16")
    cu = x["cu_seqlens"]
    # reference with the library's own hipMalloc
    hctx = mf.Context(0, allocator="hip")
    ref_store = mf.compress(Q, K, tau, wl.B, cu_seqlens=cu, ctx=hctx)
    ref_O = mf.retrieve(ref_store, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    ref_host = ref_store.to_host()

    al = _Budget(1 << 40)
    ctx = mf.Context(0, allocator=(al.alloc, al.free))
    store = mf.compress(Q, K, tau, wl.B, cu_seqlens=cu, ctx=ctx)
    O = mf.retrieve(store, W, V, x["kv_head_map"])
    torch.cuda.synchronize()
    assert al.taken > 0 and torch.equal(O, ref_O)
    host = store.to_host()
    for key in ["block_ptr", "block_idx", "probs_bits", "row_kept_mass"]:
        assert np.array_equal(host[key], ref_host[key]), key
    held = dict(al.live)

    # a store larger than the budget allows: MF_ERR_OOM, nothing new stays allocated
    al.budget = sum(al.live.values()) + (1 << 20)
    with pytest.raises(mf.MapflowError, match="OOM"):
        mf.BlockStore.create(16, wl.B, cu, capacity=10 ** 6, ctx=ctx)
    assert al.live == held and al.refused >= 1
    # the same in the middle of a compress: scratch for a longer sequence cannot grow
    big = synth.make_layer_inputs(wl, 24, lengths=[4000], H_s=16, H_r=12, H_kv=4, d=128)
    Qb, Kb = to_dev(big["q_s"], "bf16"), to_dev(big["k_s"], "bf16")
    al.budget = 1 << 40
    sb = mf.BlockStore.create(16, wl.B, [0, 4000], ctx=ctx)
    al.budget = sum(al.live.values()) + (1 << 20)
    n_live = len(al.live)
    with pytest.raises(mf.MapflowError, match="OOM"):
        mf.compress_into(sb, Qb, Kb, tau)
    assert len(al.live) <= n_live                       # at most the old scratch was handed back
    # with room again the same call succeeds and matches the hipMalloc context
    al.budget = 1 << 40
    mf.compress_into(sb, Qb, Kb, tau)
    n = sb.sync()
    ref_b = mf.compress(Qb, Kb, tau, wl.B, ctx=hctx)
    torch.cuda.synchronize()
    assert n == ref_b.raw.nnzb
    assert np.array_equal(sb.to_host()["probs_bits"], ref_b.to_host()["probs_bits"])
    # everything goes back: stores, prepared V, scratch
    for obj in (store, sb):
        obj.free()
    ctx.close()
    assert al.live == {}, f"{len(al.live)} buffers still held"
    assert al.taken == al.given
    ref_store.free()
    ref_b.free()
    hctx.close()


@pytest.mark.parametrize("k", range(6))
def test_prefill_pipeline_random_depths(mf, k):
    """Seeded depths, ring sizes and recomputed-layer counts (including no recomputed layer and a
    ring as deep as the mapped layers): every layer of both schedules equals the one-stream serial
    run bit for bit."""
    r = np.random.default_rng(np.random.SeedSequence([4949, k]))
    n_recv = int(r.integers(2, 8))
    n_send = int(r.integers(2, 10))
    R = 0 if k == 0 else int(r.integers(0, n_recv))       # case 0: no recomputed layer
    n_map = n_recv - R
    n_slots = int(r.integers(1, n_map + 1))
    L = int(r.integers(70, 400))
    H_s, H_r, H_kv, d = 8, 6, 2, 64
    pi, send, recv, kv, tau, B = _pipeline_case(L, n_send, n_recv, R, H_s, H_r, H_kv, d, seed=60 + k)
    say(f"case: random pipeline {k}: L={L} pi={pi} slots={n_slots}")
    dsend, drecv = _to_device(send, recv)
    cu = [0, L]
    mf.map_layers(pi, n_send, R)
    slots = [mf.BlockStore.create(H_s, B, cu) for _ in range(n_slots)]
    s_main, s_pre = torch.cuda.Stream(), torch.cuda.Stream()
    serial = {}
    for l in range(n_recv):
        rr = drecv[l]
        if pi[l] < 0:
            serial[l] = mf.dense_attention(rr["q"], rr["k"], rr["v"], kv, cu_seqlens=cu)
        else:
            st = mf.BlockStore.create(H_s, B, cu)
            mf.compress_into(st, *dsend[pi[l]], tau)
            serial[l] = mf.retrieve_prepared(st, rr["w"], mf.v_prepare(rr["v"], B, cu), kv)
    torch.cuda.synchronize()
    for isolate in (True, False):
        O = _outs(recv, L, H_r, d)
        for rr, o in zip(drecv, O):
            rr["o"] = o
        torch.cuda.current_stream().synchronize()
        mf.prefill_layers(slots, dsend, drecv, kv, tau, isolate=isolate, stream_main=s_main, stream_prefetch=s_pre)
        s_main.synchronize()
        for l in range(n_recv):
            assert torch.equal(O[l], serial[l]), f"isolate={isolate}: layer {l}"
