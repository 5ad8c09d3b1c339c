"""GPU test of mf_retrieve_noalloc, the retrieve that allocates no device memory: through the C ABI
it must give mf_retrieve's output bit for bit, on two calls in a row (the second with a smaller
input, so stale contents of the shared fixed array would show), for contiguous and paged V, and it
must not call the context's allocator.  Sizes past its fixed array are refused before any launch."""
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


class _Counting:
    def __init__(self):
        self.calls = 0

    def alloc(self, nbytes, stream):
        self.calls += 1
        return torch.cuda.caching_allocator_alloc(int(nbytes), 0, int(stream or 0))

    def free(self, ptr, nbytes, stream):
        torch.cuda.caching_allocator_delete(ptr)


def _case(mf, ctx, wl, seed, lengths, H_s, H_r, H_kv, d, paged):
    x = synth.make_layer_inputs(wl, seed, lengths=lengths, H_s=H_s, H_r=H_r, H_kv=H_kv, d=d)
    tau = float(np.float32(wl.tau))
    Q, K = to_dev(x["q_s"], "bf16"), to_dev(x["k_s"], "bf16")
    store = mf.compress(Q, K, tau, wl.B, cu_seqlens=x["cu_seqlens"], ctx=ctx)
    W = to_dev(x["w"])
    kw = {}
    if paged:
        table, n_pages = synth.make_page_table(lengths, 16, seed=seed)
        V = to_dev(synth.page_v(x["v_r"], lengths, table, 16, n_pages), "bf16")
        kw = dict(page_table=torch.from_numpy(table).cuda(), page_size=16)
    else:
        V = to_dev(x["v_r"], "bf16")
    return x, store, W, V, kw


def test_retrieve_noalloc_equals_retrieve_and_allocates_nothing(mf):
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    al = _Counting()
    ctx = mf.Context(0, allocator=(al.alloc, al.free))
    cases = [
        dict(seed=31, lengths=[700, 300], H_s=32, H_r=24, H_kv=8, d=128, paged=False),
        dict(seed=32, lengths=[200, 1, 90], H_s=16, H_r=12, H_kv=4, d=64, paged=True),   # smaller
    ]
    for c in cases:
        say(f"case: retrieve_noalloc {c}")
        x, store, W, V, kw = _case(mf, ctx, wl, **c)
        ref = mf.retrieve(store, W, V, x["kv_head_map"], **kw)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        before = al.calls
        mf.retrieve_noalloc(store, W, V, x["kv_head_map"], out=out, **kw)
        torch.cuda.synchronize()
        assert al.calls == before, "the no-allocation retrieve called the allocator"
        assert torch.equal(out, ref), "differs from mf_retrieve"
        host = store.to_host()
        gs = gpu_store_for_oracle(host, x["cu_seqlens"], wl.B, c["H_s"])
        v_or = x["v_r"]
        assert_out_close(out.cpu().numpy(), oracle.retrieve(gs, x["w"], v_or, x["kv_head_map"]), "O_r (no alloc)")
    ctx.close()


@pytest.mark.parametrize("k", range(6))
def test_retrieve_noalloc_random_shapes(mf, k):
    """Seeded shapes within the array's limit (contiguous or paged V): the allocation-free
    retrieve equals mf_retrieve bit for bit and calls no allocator."""
    r = np.random.default_rng(np.random.SeedSequence([5151, k]))
    wl = synth.WORKLOADS["pair_8b3b_8k"]
    H_r = int(r.integers(1, 49))
    c = dict(seed=40 + k, lengths=[int(n) for n in r.integers(1, 700, size=int(r.integers(1, 4)))],
             H_s=int(r.integers(1, 65)), H_r=H_r,
             H_kv=int(r.choice([h for h in range(1, H_r + 1) if H_r % h == 0])),
             d=int(r.choice([64, 128])), paged=bool(r.integers(0, 2)))
    al = _Counting()
    ctx = mf.Context(0, allocator=(al.alloc, al.free))
    say(f"case: random retrieve_noalloc {k}: {c}")
    x, store, W, V, kw = _case(mf, ctx, wl, **c)
    ref = mf.retrieve(store, W, V, x["kv_head_map"], **kw)
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    before = al.calls
    mf.retrieve_noalloc(store, W, V, x["kv_head_map"], out=out, **kw)
    torch.cuda.synchronize()
    assert al.calls == before, "the no-allocation retrieve called the allocator"
    assert torch.equal(out, ref), "differs from mf_retrieve"
    del store
    ctx.close()


def test_retrieve_noalloc_refuses_sizes_past_its_array(mf):
    H_s, B, T, H_kv, d = 8, 64, 32768 + 64, 8, 128          # one block row too many
    store = mf.BlockStore.create(H_s, B, [0, T], capacity=0)
    W = torch.full((8, H_s), 1.0 / H_s, device="cuda")
    V = torch.zeros((T, H_kv, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, 8, d), 7.0, device="cuda")
    with pytest.raises(mf.MapflowError, match="UNSUPPORTED"):
        mf.retrieve_noalloc(store, W, V, [g for g in range(8)], out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "output written by a refused call"
