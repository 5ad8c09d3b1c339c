// C ABI of libmapflow: argument validation, geometry of packed batches, context scratch memory,
// block-store allocation, and dispatch to the kernels.  See include/mapflow.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/mapflow.h"
#include "kernels.h"

#define MF_EXPORT __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

mf_status fail(mf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

mf_status hip_fail(hipError_t e, const char* what) {
  return fail(MF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MF_HIP(call, what)                      \
  do {                                          \
    hipError_t _e = (call);                     \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// ---- geometry of a packed batch cut into B-token block rows ------------------------------------
struct Geometry {
  int B = 0, n_seq = 0, n_brow = 0, nb_max = 0;
  int64_t T = 0, n_causal = 0;
  std::vector<int32_t> info;      // [n_brow][4]
  std::vector<int32_t> order;     // block rows by descending in-sequence index
  std::vector<int32_t> brow_seq;  // [n_brow]
  std::vector<int32_t> coff;      // [n_brow] causal blocks of all earlier block rows
  std::vector<int32_t> pairs;     // [n_pair][2] block rows (I, I+1) of one sequence (-1: none)
  std::vector<int32_t> cu;        // copy of cu_seqlens
  std::vector<int32_t> row_begin; // [n_seq] first block row compressed / retrieved per sequence
  std::vector<uint8_t> active;    // [n_brow] row >= its sequence's row_begin
  int n_pair = 0;
  int n_order = 0;                // active rows (the entries of order)
  bool ranged = false;            // some row_begin > 0
};

// Block-row geometry of a packed batch.  row_begin (per sequence, NULL = all 0) restricts the rows
// that are compressed and retrieved to I >= row_begin[s] (chunked prefill); every row still
// exists as a key block row.
mf_status build_geometry(const int32_t* cu, int32_t n_seq, int32_t B, Geometry& g,
                         const int32_t* row_begin = nullptr) {
  if (cu == nullptr) return fail(MF_ERR_INVALID, "cu_seqlens_host is NULL");
  if (n_seq < 1) return fail(MF_ERR_INVALID, "n_seq must be >= 1 (got %d)", n_seq);
  if (B != 16 && B != 32 && B != 64 && B != 128)
    return fail(MF_ERR_INVALID, "block size B must be 16, 32, 64 or 128 (got %d)", B);
  if (cu[0] != 0) return fail(MF_ERR_INVALID, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  g = Geometry();
  g.B = B;
  g.n_seq = n_seq;
  g.cu.assign(cu, cu + n_seq + 1);
  for (int s = 0; s < n_seq; ++s) {
    if (cu[s + 1] < cu[s])
      return fail(MF_ERR_INVALID, "cu_seqlens must be non-decreasing (entry %d)", s + 1);
    const int n = cu[s + 1] - cu[s];
    const int nb = (n + B - 1) / B;
    const int rb = row_begin ? row_begin[s] : 0;
    if (rb < 0 || rb > nb)
      return fail(MF_ERR_INVALID, "row_begin[%d] = %d outside [0, %d]", s, rb, nb);
    g.row_begin.push_back(rb);
    g.ranged |= rb > 0;
    g.nb_max = std::max(g.nb_max, nb);
    g.n_causal += (int64_t)nb * (nb + 1) / 2;
    for (int I = 0; I < nb; ++I) {
      g.info.insert(g.info.end(), {cu[s] + I * B, cu[s], n, I});
      g.brow_seq.push_back(s);
      g.active.push_back(I >= rb ? 1 : 0);
      g.coff.push_back((int32_t)std::min<int64_t>(g.n_causal - (int64_t)nb * (nb + 1) / 2 + (int64_t)I * (I + 1) / 2,
                                                  INT32_MAX));
    }
  }
  g.T = cu[n_seq];
  g.n_brow = (int)g.brow_seq.size();
  for (int b = 0; b < g.n_brow; ++b)
    if (g.active[b]) g.order.push_back(b);
  g.n_order = (int)g.order.size();
  std::stable_sort(g.order.begin(), g.order.end(), [&](int x, int y) {
    return g.info[4 * x + 3] > g.info[4 * y + 3];
  });
  // pairs of consecutive active block rows of one sequence (from its first active row), the one
  // with the larger row first
  std::vector<std::pair<int, int>> pr;
  for (int b = 0; b < g.n_brow; ++b) {
    if (!g.active[b] || (g.info[4 * b + 3] - g.row_begin[g.brow_seq[b]]) % 2 != 0) continue;
    const bool has_next = b + 1 < g.n_brow && g.brow_seq[b + 1] == g.brow_seq[b];
    pr.emplace_back(b, has_next ? b + 1 : -1);
  }
  auto top = [&](const std::pair<int, int>& x) { return g.info[4 * (x.second >= 0 ? x.second : x.first) + 3]; };
  std::stable_sort(pr.begin(), pr.end(), [&](const auto& x, const auto& y) { return top(x) > top(y); });
  g.n_pair = (int)pr.size();
  for (const auto& x : pr) g.pairs.insert(g.pairs.end(), {x.first, x.second});
  if (g.n_causal >= (int64_t)INT32_MAX)
    return fail(MF_ERR_UNSUPPORTED, "more than 2^31 causal blocks (%lld)", (long long)g.n_causal);
  return MF_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Where device memory comes from: the caller's allocator, or hipMalloc / hipFree.  Stores and
// prepared V keep a copy, so they can be released after their context is gone.
struct Allocator {
  mf_alloc_fn alloc = nullptr;
  mf_free_fn release = nullptr;
  void* user = nullptr;

  void* take(size_t bytes, hipStream_t s) const {
    if (alloc) return alloc(bytes, s, user);
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return p;
  }
  // Callers have made sure no enqueued work still reads or writes p.
  void give(void* p, size_t bytes, hipStream_t s) const {
    if (!p) return;
    if (release) release(p, bytes, s, user);
    else (void)hipFree(p);
  }
};

// One device buffer that only grows.
struct Scratch {
  void* p = nullptr;
  size_t bytes = 0;
};

// Grow a context buffer.  Every user of one buffer is ordered on the calling stream (the
// context's contract), so once that stream is idle the old buffer is unused.
mf_status ensure(const Allocator& al, Scratch& s, size_t bytes, const char* what, hipStream_t stream) {
  if (bytes <= s.bytes) return MF_OK;
  if (s.p) {
    MF_HIP(hipStreamSynchronize(stream), "hipStreamSynchronize before scratch growth");
    al.give(s.p, s.bytes, stream);
    s.p = nullptr;
    s.bytes = 0;
  }
  const size_t want = align_up(bytes, 1 << 20);
  s.p = al.take(want, stream);
  if (!s.p) return fail(MF_ERR_OOM, "out of device memory growing %s scratch to %zu bytes", what, want);
  s.bytes = want;
  return MF_OK;
}

void release_scratch(const Allocator& al, Scratch& s) {
  al.give(s.p, s.bytes, nullptr);
  s = Scratch();
}

// Bookkeeping behind mf_bsr::_owner.
struct BsrOwner {
  Allocator al;
  void* meta = nullptr;
  size_t meta_bytes = 0;
  void* data = nullptr;
  size_t data_bytes = 0;
  int32_t* pairs = nullptr;       // device copy of geom.pairs (inside meta)
  uint8_t* active = nullptr;      // device copy of geom.active when the store is ranged (inside meta)
  int32_t* brow_seq = nullptr;    // device copy of geom.brow_seq (inside meta)
  int32_t* gorder = nullptr;      // the gather's row order (inside meta), see gather_order
  bool cache_owned = false;       // an entry of an mf_cache: freed by the cache only
  Geometry geom;
};

// Bookkeeping behind mf_vfrag::_owner.
struct VfragOwner {
  Allocator al;
  void* tables = nullptr;   // info, brow_seq, exps, vmax scratch
  size_t tables_bytes = 0;
  void* frag = nullptr;     // only when the library allocated it
  size_t frag_bytes = 0;
  int32_t* info = nullptr;
  int32_t* brow_seq = nullptr;
  uint32_t* vmax = nullptr;
  Geometry geom;
};

// Events and timings of mf_prefill_layers.
struct PrefillState {
  std::vector<hipEvent_t> ev;   // created on demand, destroyed with the context
  int n_map = 0, R = 0;
  bool timed = false;           // the last call recorded timing events
  // event indices of the last call
  int e_start = 0, e_end = 0;
  std::vector<int> d0, d1, c0, c1, v0, r0, r1;
};

}  // namespace

struct mf_ctx {
  int device = 0;
  Allocator al;
  Scratch lse2, Mh, M, flags, counts, part, zbuf, ktile, hflags, lse2n, den;
  mf_vfrag vf_retrieve{};   // context-owned prepared V (mf_retrieve)
  mf_vfrag vf_dense{};      // context-owned prepared V (mf_dense_attention)
  mf_vfrag vf_prefill{};    // context-owned prepared sender V (mf_compress_prefill_into)
  mf_vfrag vf_pipe{};       // context-owned prepared receiver V (mf_prefill_layers)
  // cached device copies of the dense-attention geometry
  Scratch dense_tables;
  std::vector<int32_t> dense_cu;
  int dense_nbrow = 0;
  // layer map installed by mf_map_layers
  std::vector<int32_t> pi;
  int n_recv = 0, n_send = 0, R = 0;
  PrefillState pre;
};

namespace {

mf_status set_device(mf_ctx* ctx) {
  if (!ctx) return fail(MF_ERR_INVALID, "context is NULL");
  MF_HIP(hipSetDevice(ctx->device), "hipSetDevice");
  return MF_OK;
}

int dtype_code(mf_dtype dt) { return dt == MF_BF16 ? mf::DT_BF16 : mf::DT_F32; }

mf_status check_dtype(mf_dtype dt) {
  if (dt != MF_F32 && dt != MF_BF16) return fail(MF_ERR_INVALID, "dtype must be MF_F32 or MF_BF16");
  return MF_OK;
}

// The gather's row order: the work order, with rows of one sequence brought together per XCD.
// The gather sends work item p to a lane of L = 8 (head groups not dividing 8: XCD p mod 8 for
// each head group) or of L = 8 / HG (each XCD serves one head group and takes the items with p
// mod L fixed), and the workgroups in flight on one XCD take consecutive items of its lane.  In a
// run of 64 L entries of the work order that holds rows of several sequences, the rows are
// grouped by sequence (work order within one), and lane x takes the x-th 64 of them: the keys
// the workgroups in flight on one XCD read then belong to one or two sequences instead of one row
// of each.  Runs of one sequence keep the work order.
std::vector<int32_t> gather_order(const Geometry& g, int H_s) {
  std::vector<int32_t> o(g.order.begin(), g.order.begin() + g.n_order);
  const int HG = (H_s + 7) / 8;
  const int L = (8 % HG == 0) ? 8 / HG : 8;
  const int R = 64 * L;
  std::vector<int32_t> run(R);
  for (int m = 0; m + R <= g.n_order; m += R) {
    bool mixed = false;
    for (int j = 1; j < R; ++j) mixed |= g.brow_seq[o[m + j]] != g.brow_seq[o[m]];
    if (!mixed) continue;
    std::copy(o.begin() + m, o.begin() + m + R, run.begin());
    std::stable_sort(run.begin(), run.end(), [&](int x, int y) { return g.brow_seq[x] < g.brow_seq[y]; });
    for (int x = 0; x < L; ++x)
      for (int k = 0; k < 64; ++k) o[m + L * k + x] = run[64 * x + k];
  }
  return o;
}

// The retrieve's row order: block row gidx runs on XCD gidx mod 8 with all its row tiles and
// head splits, and about 8 block rows are in flight per XCD.  In each run of 8 K entries of the
// work order XCD x takes K consecutive entries (x-th from the front in even runs, from the back
// in odd runs, so that no XCD always gets the longest rows of a run): the rows in flight on an
// XCD are then neighbours, whose kept blocks and V tiles overlap most.
std::vector<int32_t> retrieve_order(const Geometry& g) {
  std::vector<int32_t> o(g.order.begin(), g.order.begin() + g.n_order);
  constexpr int K = 8, R = 8 * K;   // 8 rows per XCD: the rows in flight on it
  for (int m = 0, run = 0; m + R <= g.n_order; m += R, ++run)
    for (int x = 0; x < 8; ++x) {
      const int src = (run & 1) ? 7 - x : x;
      for (int k = 0; k < K; ++k) o[m + 8 * k + x] = g.order[m + K * src + k];
    }
  return o;
}

// The statistics' pair order, grouped the same way: with a multiple of 8 heads every XCD takes
// the pairs in order (L = 1), else XCD b mod 8 takes every 8th (L = 8); in a run of 256 L pairs of
// several sequences, the pairs are grouped by sequence and lane x takes the x-th 256.
std::vector<int32_t> stats_pairs(const Geometry& g, int H_s) {
  std::vector<int32_t> o(g.pairs.begin(), g.pairs.begin() + 2 * (size_t)g.n_pair);
  const int L = (H_s % 8 == 0) ? 1 : 8;
  const int R = 256 * L;
  auto seq = [&](int i) { return g.brow_seq[o[2 * i]]; };
  std::vector<std::pair<int32_t, int32_t>> run(R);
  for (int m = 0; m + R <= g.n_pair; m += R) {
    bool mixed = false;
    for (int j = 1; j < R; ++j) mixed |= seq(m + j) != seq(m);
    if (!mixed) continue;
    for (int j = 0; j < R; ++j) run[j] = {o[2 * (m + j)], o[2 * (m + j) + 1]};
    std::stable_sort(run.begin(), run.end(), [&](const auto& x, const auto& y) {
      return g.brow_seq[x.first] < g.brow_seq[y.first];
    });
    for (int x = 0; x < L; ++x)
      for (int k = 0; k < 256; ++k) {
        const int i = m + L * k + x;
        o[2 * i] = run[256 * x + k].first;
        o[2 * i + 1] = run[256 * x + k].second;
      }
  }
  return o;
}

mf_status alloc_bsr_meta(const Geometry& g, int H_s, mf_bsr* out, BsrOwner* own) {
  const size_t n_info = (size_t)g.n_brow * 4 * 4;
  const size_t o_info = 0;
  const size_t o_order = align_up(o_info + n_info, 256);
  const size_t o_gorder = align_up(o_order + (size_t)g.n_brow * 4, 256);
  const size_t o_coff = align_up(o_gorder + (size_t)g.n_brow * 4, 256);
  const size_t o_seq = align_up(o_coff + (size_t)g.n_brow * 4, 256);
  const size_t o_ptr = align_up(o_seq + (size_t)g.n_brow * 4, 256);
  const size_t o_rkm = align_up(o_ptr + (size_t)(g.n_brow + 1) * 4, 256);
  const size_t o_cnt = align_up(o_rkm + (size_t)H_s * g.T * 4, 256);
  const size_t o_pairs = o_cnt + 256;
  const size_t o_active = align_up(o_pairs + (size_t)g.n_pair * 8, 256);
  const size_t total = align_up(o_active + (size_t)g.n_brow, 256) + 256;
  own->meta = own->al.take(total, nullptr);
  if (!own->meta) return fail(MF_ERR_OOM, "out of device memory for block-store metadata (%zu bytes)", total);
  own->meta_bytes = total;
  char* base = static_cast<char*>(own->meta);
  out->brow_info = reinterpret_cast<int32_t*>(base + o_info);
  out->brow_order = reinterpret_cast<int32_t*>(base + o_order);
  out->brow_coff = reinterpret_cast<int32_t*>(base + o_coff);
  out->block_ptr = reinterpret_cast<int32_t*>(base + o_ptr);
  out->row_kept_mass = reinterpret_cast<float*>(base + o_rkm);
  out->counters = reinterpret_cast<int32_t*>(base + o_cnt);
  own->brow_seq = reinterpret_cast<int32_t*>(base + o_seq);
  own->gorder = reinterpret_cast<int32_t*>(base + o_gorder);
  own->pairs = reinterpret_cast<int32_t*>(base + o_pairs);
  own->active = g.ranged ? reinterpret_cast<uint8_t*>(base + o_active) : nullptr;
  out->n_order = g.n_order;
  hipError_t e = hipSuccess;
  if (g.n_brow > 0) {
    e = hipMemcpy(out->brow_info, g.info.data(), n_info, hipMemcpyHostToDevice);
    // the order lists the active rows only (n_order <= n_brow entries; none past them are read)
    if (e == hipSuccess && g.n_order > 0) {
      const std::vector<int32_t> ro = retrieve_order(g);
      e = hipMemcpy(out->brow_order, ro.data(), (size_t)g.n_order * 4, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && g.n_order > 0) {
      const std::vector<int32_t> go = gather_order(g, H_s);
      e = hipMemcpy(own->gorder, go.data(), (size_t)g.n_order * 4, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess)
      e = hipMemcpy(out->brow_coff, g.coff.data(), (size_t)g.n_brow * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(own->brow_seq, g.brow_seq.data(), (size_t)g.n_brow * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess && g.n_pair > 0) {
      const std::vector<int32_t> sp = stats_pairs(g, H_s);
      e = hipMemcpy(own->pairs, sp.data(), (size_t)g.n_pair * 8, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && own->active)
      e = hipMemcpy(own->active, g.active.data(), (size_t)g.n_brow, hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipMemset(out->block_ptr, 0, (size_t)(g.n_brow + 1) * 4);
  if (e == hipSuccess) e = hipMemset(out->counters, 0, 256);
  if (e == hipSuccess && g.T > 0) e = hipMemset(out->row_kept_mass, 0, (size_t)H_s * g.T * 4);
  // the initialisation is complete before any stream can use the store, and before a failed
  // creation hands the memory back
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipDeviceSynchronize();
    own->al.give(own->meta, own->meta_bytes, nullptr);
    own->meta = nullptr;
    return hip_fail(e, "initialising block-store metadata");
  }
  return MF_OK;
}

size_t probs_block_bytes(int H_s, int B) { return (size_t)((H_s + 7) / 8) * B * B * 8 * 2; }

mf_status alloc_bsr_data(int64_t capacity, int H_s, int B, mf_bsr* out, BsrOwner* own) {
  const size_t o_idx = 0;
  const size_t o_row = align_up((size_t)capacity * 4, 256);
  const size_t o_probs = align_up(o_row + (size_t)capacity * 4, 256);
  const size_t total = o_probs + (size_t)capacity * probs_block_bytes(H_s, B) + 256;
  own->data = own->al.take(total, nullptr);
  if (!own->data)
    return fail(MF_ERR_OOM, "out of device memory for %lld kept blocks (%zu bytes)", (long long)capacity, total);
  own->data_bytes = total;
  char* base = static_cast<char*>(own->data);
  out->block_idx = reinterpret_cast<int32_t*>(base + o_idx);
  out->block_row = reinterpret_cast<int32_t*>(base + o_row);
  out->probs = reinterpret_cast<uint16_t*>(base + o_probs);
  out->capacity = capacity;
  return MF_OK;
}

// Hand back a store's device arrays (the device must be idle for them).
void bsr_release_arrays(BsrOwner* own) {
  own->al.give(own->meta, own->meta_bytes, nullptr);
  own->al.give(own->data, own->data_bytes, nullptr);
  own->meta = own->data = nullptr;
  own->meta_bytes = own->data_bytes = 0;
}

// Q, K and V are read with 16-byte loads (and key tiles by 16-byte DMA), so their base pointers
// must be 16-byte aligned (every row of a contiguous layout then is, since d * size >= 128).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

mf_status validate_compress(const void* Q, const void* K, mf_dtype dtype, int32_t d, float tau,
                            const mf_bsr* bsr) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL or not created by mf_bsr_create");
  if (!Q || !K) return fail(MF_ERR_INVALID, "Q or K is NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(MF_ERR_INVALID, "Q and K must be 16-byte aligned");
  mf_status st = check_dtype(dtype);
  if (st != MF_OK) return st;
  if (d != 64 && d != 128) return fail(MF_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
  if (!(tau > 0.f && tau <= 1.f)) return fail(MF_ERR_INVALID, "tau must be in (0, 1] (got %g)", (double)tau);
  if (!mf::compress_supported(dtype_code(dtype), bsr->B, d))
    return fail(MF_ERR_UNSUPPORTED, "no compress kernel for B=%d d=%d", bsr->B, d);
  if (bsr->nb_max > 4096)
    return fail(MF_ERR_UNSUPPORTED, "sequence too long for the selection kernel (%d blocks > 4096)", bsr->nb_max);
  return MF_OK;
}

mf_status prepare_compress_args(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype,
                                int32_t d, float tau, mf_bsr* bsr, int64_t capacity,
                                mf::CompressArgs& a, hipStream_t stream) {
  const size_t nbn = (size_t)bsr->n_brow * bsr->nb_max;
  mf_status st;
  if ((st = ensure(ctx->al, ctx->lse2, (size_t)bsr->H_s * bsr->T * 4 + 256, "lse", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->zbuf, (size_t)bsr->H_s * bsr->n_causal * bsr->B * 8 + 256, "block statistics", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->Mh, (size_t)bsr->H_s * nbn * 4 + 256, "block mass", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->M, nbn * 8 + 256, "head-summed mass", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->flags, nbn + 256, "flags", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->counts, (size_t)bsr->n_brow * 4 + 256, "counts", stream)) != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->part, (size_t)bsr->n_brow * ((bsr->nb_max + mf::kGatherChunk - 1) / mf::kGatherChunk) * bsr->H_s * bsr->B * 8 + 256,
                   "row sums", stream)) != MF_OK)
    return st;
  const size_t elem = dtype == MF_BF16 ? 2 : 4;
  if ((st = ensure(ctx->al, ctx->ktile, (size_t)bsr->H_s * bsr->n_brow * bsr->B * d * elem + 256, "key operand tiles", stream)) != MF_OK)
    return st;
  a = mf::CompressArgs{};
  a.Q = Q;
  a.K = K;
  a.dtype = dtype_code(dtype);
  a.H_s = bsr->H_s;
  a.d = d;
  a.B = bsr->B;
  a.T = bsr->T;
  a.n_brow = bsr->n_brow;
  a.nb_max = bsr->nb_max;
  a.info = bsr->brow_info;
  a.order = static_cast<const BsrOwner*>(bsr->_owner)->gorder;
  a.coff = bsr->brow_coff;
  a.pairs = static_cast<const BsrOwner*>(bsr->_owner)->pairs;
  a.n_pair = static_cast<const BsrOwner*>(bsr->_owner)->geom.n_pair;
  a.active = static_cast<const BsrOwner*>(bsr->_owner)->active;
  a.n_order = bsr->n_order;
  a.n_causal = bsr->n_causal;
  a.tau = (double)tau;
  a.scale2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  a.lse2 = static_cast<float*>(ctx->lse2.p);
  a.zbuf = static_cast<float2*>(ctx->zbuf.p);
  a.Mh = static_cast<float*>(ctx->Mh.p);
  a.M = static_cast<double*>(ctx->M.p);
  a.flags = static_cast<uint8_t*>(ctx->flags.p);
  a.counts = static_cast<int32_t*>(ctx->counts.p);
  a.part = static_cast<double*>(ctx->part.p);
  a.ktile = ctx->ktile.p;
  a.block_ptr = bsr->block_ptr;
  a.block_idx = bsr->block_idx;
  a.block_row = bsr->block_row;
  a.probs = bsr->probs;
  a.rkm = bsr->row_kept_mass;
  a.counters = bsr->counters;
  a.capacity = capacity;
  return MF_OK;
}

mf_status build_headmap(const int32_t* kvmap, int H, int H_kv, mf::HeadMap& hm) {
  if (!kvmap) return fail(MF_ERR_INVALID, "kv_head_map_host is NULL");
  if (H < 1 || H > 64) return fail(MF_ERR_UNSUPPORTED, "head count %d outside [1, 64]", H);
  std::memset(&hm, 0, sizeof(hm));
  std::vector<int> perm(H);
  for (int g = 0; g < H; ++g) {
    if (kvmap[g] < 0 || kvmap[g] >= H_kv)
      return fail(MF_ERR_INVALID, "kv_head_map[%d] = %d outside [0, %d)", g, kvmap[g], H_kv);
    hm.kv[g] = (int8_t)kvmap[g];
    perm[g] = g;
  }
  std::stable_sort(perm.begin(), perm.end(), [&](int x, int y) { return kvmap[x] < kvmap[y]; });
  for (int g = 0; g < H; ++g) hm.perm[g] = (int8_t)perm[g];
  return MF_OK;
}

mf_status vfrag_prepare(mf_ctx* ctx, const int32_t* cu, int32_t n_seq, int32_t B, const void* V,
                        mf_dtype dtype, int32_t H_kv, int32_t d, const int32_t* page_table,
                        int32_t page_size, int32_t pages_per_seq, mf_vfrag* out, bool reuse,
                        hipStream_t stream) {
  if (!out) return fail(MF_ERR_INVALID, "output vfrag is NULL");
  if (!V) return fail(MF_ERR_INVALID, "V is NULL");
  if (!aligned16(V)) return fail(MF_ERR_INVALID, "V must be 16-byte aligned");
  mf_status st = check_dtype(dtype);
  if (st != MF_OK) return st;
  if (d != 64 && d != 128) return fail(MF_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
  if (H_kv < 1 || H_kv > 64) return fail(MF_ERR_INVALID, "H_kv must be in [1, 64] (got %d)", H_kv);
  if (B != 32 && B != 64) return fail(MF_ERR_UNSUPPORTED, "V preparation supports B = 32 or 64 (got %d)", B);
  if (page_table && (page_size < 1 || pages_per_seq < 1))
    return fail(MF_ERR_INVALID, "paged V needs page_size >= 1 and pages_per_seq >= 1");
  Geometry g;
  if ((st = build_geometry(cu, n_seq, B, g)) != MF_OK) return st;
  if (page_table)
    for (int s = 0; s < n_seq; ++s)
      if ((int64_t)(cu[s + 1] - cu[s]) > (int64_t)page_size * pages_per_seq)
        return fail(MF_ERR_INVALID, "sequence %d needs more than pages_per_seq pages", s);

  VfragOwner* own = static_cast<VfragOwner*>(out->_owner);
  const bool same_geom = own && own->geom.cu == g.cu && own->geom.B == B && out->H_kv == H_kv && out->d == d;
  if (!(reuse && same_geom)) {
    if (own) {
      // a context-owned buffer of another geometry: its users are ordered on this stream
      if (reuse) MF_HIP(hipStreamSynchronize(stream), "hipStreamSynchronize before V scratch growth");
      own->al.give(own->tables, own->tables_bytes, stream);
      own->al.give(own->frag, own->frag_bytes, stream);
      delete own;
      out->_owner = nullptr;
      if (reuse) out->frag = nullptr;
    }
    own = new (std::nothrow) VfragOwner();
    if (!own) return fail(MF_ERR_OOM, "host allocation failed");
    own->al = ctx->al;
    const size_t o_info = 0;
    const size_t o_seq = align_up((size_t)g.n_brow * 16, 256);
    const size_t o_exp = align_up(o_seq + (size_t)g.n_brow * 4, 256);
    const size_t o_max = align_up(o_exp + (size_t)H_kv * 4, 256);
    const size_t tb = o_max + 256;
    own->tables = own->al.take(tb, stream);
    if (!own->tables) {
      delete own;
      return fail(MF_ERR_OOM, "out of device memory for V tables");
    }
    own->tables_bytes = tb;
    char* base = static_cast<char*>(own->tables);
    own->info = reinterpret_cast<int32_t*>(base + o_info);
    own->brow_seq = reinterpret_cast<int32_t*>(base + o_seq);
    own->vmax = reinterpret_cast<uint32_t*>(base + o_max);
    hipError_t e = hipSuccess;
    if (g.n_brow > 0) {
      e = hipMemcpy(own->info, g.info.data(), (size_t)g.n_brow * 16, hipMemcpyHostToDevice);
      if (e == hipSuccess)
        e = hipMemcpy(own->brow_seq, g.brow_seq.data(), (size_t)g.n_brow * 4, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
      (void)hipDeviceSynchronize();
      own->al.give(own->tables, own->tables_bytes, stream);
      delete own;
      return hip_fail(e, "uploading V tables");
    }
    if (out->frag == nullptr) {
      const size_t fb = (size_t)H_kv * g.n_brow * B * d * 2 + 256;
      own->frag = own->al.take(fb, stream);
      if (!own->frag) {
        own->al.give(own->tables, own->tables_bytes, stream);
        delete own;
        return fail(MF_ERR_OOM, "out of device memory for prepared V (%zu bytes)", fb);
      }
      own->frag_bytes = fb;
      out->frag = static_cast<uint16_t*>(own->frag);
    }
    out->exps = reinterpret_cast<int32_t*>(base + o_exp);
    own->geom = g;
    out->_owner = own;
  }
  out->B = B;
  out->d = d;
  out->H_kv = H_kv;
  out->n_brow = g.n_brow;
  out->T = g.T;
  if (g.n_brow == 0) return MF_OK;
  mf::VprepArgs va{};
  va.V = V;
  va.dtype = dtype_code(dtype);
  va.H_kv = H_kv;
  va.d = d;
  va.B = B;
  va.T = g.T;
  va.n_brow = g.n_brow;
  va.info = own->info;
  va.page_table = page_table;
  va.page_size = page_size;
  va.pages_per_seq = pages_per_seq;
  va.brow_seq = own->brow_seq;
  va.vmax_bits = own->vmax;
  va.frag = out->frag;
  va.exps = out->exps;
  MF_HIP(mf::v_prepare(va, stream), "V preparation launch");
  return MF_OK;
}

// Release a prepared V (the device must be idle for it).
void vfrag_release(mf_vfrag* vf) {
  if (!vf) return;
  VfragOwner* own = static_cast<VfragOwner*>(vf->_owner);
  if (own) {
    own->al.give(own->tables, own->tables_bytes, nullptr);
    own->al.give(own->frag, own->frag_bytes, nullptr);
    delete own;
  }
  std::memset(vf, 0, sizeof(*vf));
}

}  // namespace

extern "C" {

MF_EXPORT const char* mf_version(void) { return "libmapflow 0.1.0 (gfx950)"; }

MF_EXPORT const char* mf_last_error(void) { return g_err.c_str(); }

MF_EXPORT mf_status mf_create(int device, mf_alloc_fn alloc, mf_free_fn release, void* user, mf_ctx** out) {
  if (!out) return fail(MF_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if ((alloc == nullptr) != (release == nullptr))
    return fail(MF_ERR_INVALID, "give both allocator callbacks or neither");
  int n = 0;
  MF_HIP(hipGetDeviceCount(&n), "hipGetDeviceCount");
  if (device < 0 || device >= n) return fail(MF_ERR_INVALID, "device %d out of range [0, %d)", device, n);
  MF_HIP(hipSetDevice(device), "hipSetDevice");
  mf_ctx* ctx = new (std::nothrow) mf_ctx();
  if (!ctx) return fail(MF_ERR_OOM, "host allocation failed");
  ctx->device = device;
  ctx->al.alloc = alloc;
  ctx->al.release = release;
  ctx->al.user = user;
  *out = ctx;
  return MF_OK;
}

MF_EXPORT mf_status mf_destroy(mf_ctx* ctx) {
  if (!ctx) return MF_OK;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  for (Scratch* s : {&ctx->lse2, &ctx->Mh, &ctx->M, &ctx->flags, &ctx->counts, &ctx->part, &ctx->zbuf, &ctx->ktile,
                     &ctx->hflags, &ctx->lse2n, &ctx->den, &ctx->dense_tables})
    release_scratch(ctx->al, *s);
  vfrag_release(&ctx->vf_retrieve);
  vfrag_release(&ctx->vf_dense);
  vfrag_release(&ctx->vf_prefill);
  vfrag_release(&ctx->vf_pipe);
  for (hipEvent_t e : ctx->pre.ev) (void)hipEventDestroy(e);
  delete ctx;
  return MF_OK;
}

MF_EXPORT mf_status mf_layer_map_uniform(int32_t n_recv, int32_t n_send, int32_t R, int32_t* pi_out) {
  if (!pi_out) return fail(MF_ERR_INVALID, "pi_out_host is NULL");
  if (n_recv < 1 || n_send < 1) return fail(MF_ERR_INVALID, "layer counts must be >= 1");
  if (R < 0 || R > n_recv) return fail(MF_ERR_INVALID, "R must be in [0, n_recv]");
  for (int l = 0; l < n_recv; ++l) {
    if (l < R) {
      pi_out[l] = -1;
    } else if (n_recv == 1) {
      pi_out[l] = 0;
    } else {
      // round(l (S-1) / (Rv-1)), halves up: floor((2 l (S-1) + (Rv-1)) / (2 (Rv-1)))
      const int64_t num = 2LL * l * (n_send - 1) + (n_recv - 1);
      pi_out[l] = (int32_t)(num / (2LL * (n_recv - 1)));
    }
  }
  return MF_OK;
}

MF_EXPORT mf_status mf_check_layer_map(const int32_t* pi, int32_t n_recv, int32_t n_send, int32_t R) {
  if (!pi) return fail(MF_ERR_INVALID, "pi_host is NULL");
  if (n_recv < 1 || n_send < 1 || R < 0 || R > n_recv) return fail(MF_ERR_INVALID, "bad layer counts");
  for (int l = 0; l < n_recv; ++l) {
    if (l < R && pi[l] != -1) return fail(MF_ERR_INVALID, "layer %d < R must map to -1", l);
    if (l >= R && (pi[l] < 0 || pi[l] >= n_send))
      return fail(MF_ERR_INVALID, "layer %d maps to %d outside [0, %d)", l, pi[l], n_send);
  }
  return MF_OK;
}

MF_EXPORT mf_status mf_map_layers(mf_ctx* ctx, const int32_t* pi, int32_t n_recv, int32_t n_send, int32_t R) {
  if (!ctx) return fail(MF_ERR_INVALID, "context is NULL");
  mf_status st = mf_check_layer_map(pi, n_recv, n_send, R);
  if (st != MF_OK) return st;
  ctx->pi.assign(pi, pi + n_recv);
  ctx->n_recv = n_recv;
  ctx->n_send = n_send;
  ctx->R = R;
  return MF_OK;
}

static mf_status bsr_create(mf_ctx* ctx, int32_t H_s, int32_t B, const int32_t* cu, int32_t n_seq,
                            const int32_t* row_begin, int64_t capacity, mf_bsr* out) {
  if (!out) return fail(MF_ERR_INVALID, "out is NULL");
  if (H_s < 1 || H_s > 64) return fail(MF_ERR_INVALID, "H_s must be in [1, 64] (got %d)", H_s);
  Geometry g;
  mf_status st = build_geometry(cu, n_seq, B, g, row_begin);
  if (st != MF_OK) return st;
  if ((st = set_device(ctx)) != MF_OK) return st;
  BsrOwner* own = new (std::nothrow) BsrOwner();
  if (!own) return fail(MF_ERR_OOM, "host allocation failed");
  own->al = ctx->al;
  mf_bsr b{};
  b.B = B;
  b.H_s = H_s;
  b.n_seq = n_seq;
  b.n_brow = g.n_brow;
  b.nb_max = g.nb_max;
  b.T = g.T;
  b.n_causal = g.n_causal;
  if (capacity < 0) {                  // every causal block of the rows that are compressed
    capacity = 0;
    for (int r = 0; r < g.n_brow; ++r)
      if (g.active[r]) capacity += g.info[4 * r + 3] + 1;
  }
  if ((st = alloc_bsr_meta(g, H_s, &b, own)) != MF_OK) {
    delete own;
    return st;
  }
  if ((st = alloc_bsr_data(capacity, H_s, B, &b, own)) != MF_OK) {
    bsr_release_arrays(own);          // the metadata initialisation finished inside alloc_bsr_meta
    delete own;
    return st;
  }
  own->geom = std::move(g);
  b._owner = own;
  *out = b;
  return MF_OK;
}

MF_EXPORT mf_status mf_bsr_create(mf_ctx* ctx, int32_t H_s, int32_t B, const int32_t* cu,
                                  int32_t n_seq, int64_t capacity, mf_bsr* out) {
  return bsr_create(ctx, H_s, B, cu, n_seq, nullptr, capacity, out);
}

MF_EXPORT mf_status mf_bsr_create_range(mf_ctx* ctx, int32_t H_s, int32_t B, const int32_t* cu,
                                        int32_t n_seq, const int32_t* row_begin, int64_t capacity,
                                        mf_bsr* out) {
  if (!row_begin) return fail(MF_ERR_INVALID, "row_begin_host is NULL");
  return bsr_create(ctx, H_s, B, cu, n_seq, row_begin, capacity, out);
}

MF_EXPORT mf_status mf_bsr_free(mf_ctx* ctx, mf_bsr* bsr) {
  if (!bsr) return MF_OK;
  BsrOwner* own = static_cast<BsrOwner*>(bsr->_owner);
  if (own && own->cache_owned) return fail(MF_ERR_INVALID, "this store belongs to a prefix cache");
  if (own) {
    if (ctx) (void)hipSetDevice(ctx->device);
    (void)hipDeviceSynchronize();       // no enqueued work may still use the arrays
    bsr_release_arrays(own);
    delete own;
  }
  std::memset(bsr, 0, sizeof(*bsr));
  return MF_OK;
}

MF_EXPORT mf_status mf_bsr_download(mf_ctx* ctx, mf_bsr* bsr, int32_t* block_ptr_host,
                                    int32_t* block_idx_host, uint16_t* probs_host,
                                    float* rkm_host) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  int32_t cnt[2] = {0, 0};
  MF_HIP(hipMemcpy(cnt, bsr->counters, sizeof(cnt), hipMemcpyDeviceToHost), "reading kept-block count");
  bsr->nnzb = std::min<int64_t>(cnt[0], bsr->capacity);
  const size_t nn = (size_t)bsr->nnzb;
  if (block_ptr_host)
    MF_HIP(hipMemcpy(block_ptr_host, bsr->block_ptr, (size_t)(bsr->n_brow + 1) * 4, hipMemcpyDeviceToHost), "copy block_ptr");
  if (block_idx_host && nn)
    MF_HIP(hipMemcpy(block_idx_host, bsr->block_idx, nn * 4, hipMemcpyDeviceToHost), "copy block_idx");
  if (probs_host && nn)
    MF_HIP(hipMemcpy(probs_host, bsr->probs, nn * probs_block_bytes(bsr->H_s, bsr->B), hipMemcpyDeviceToHost), "copy probs");
  if (rkm_host && bsr->T)
    MF_HIP(hipMemcpy(rkm_host, bsr->row_kept_mass, (size_t)bsr->H_s * bsr->T * 4, hipMemcpyDeviceToHost), "copy row_kept_mass");
  return MF_OK;
}

MF_EXPORT mf_status mf_bsr_download_blocks(mf_ctx* ctx, mf_bsr* bsr, int64_t first, int64_t count,
                                           int32_t* block_idx_host, uint16_t* probs_host) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  int32_t cnt[2] = {0, 0};
  MF_HIP(hipMemcpy(cnt, bsr->counters, sizeof(cnt), hipMemcpyDeviceToHost), "reading kept-block count");
  bsr->nnzb = std::min<int64_t>(cnt[0], bsr->capacity);
  if (first < 0 || count < 0 || first + count > bsr->nnzb)
    return fail(MF_ERR_INVALID, "blocks [%lld, %lld) outside the %lld kept blocks", (long long)first,
                (long long)(first + count), (long long)bsr->nnzb);
  if (count == 0) return MF_OK;
  if (block_idx_host)
    MF_HIP(hipMemcpy(block_idx_host, bsr->block_idx + first, (size_t)count * 4, hipMemcpyDeviceToHost), "copy block_idx");
  if (probs_host) {
    const size_t bb = probs_block_bytes(bsr->H_s, bsr->B);
    MF_HIP(hipMemcpy(probs_host, reinterpret_cast<const unsigned char*>(bsr->probs) + (size_t)first * bb,
                     (size_t)count * bb, hipMemcpyDeviceToHost), "copy probs");
  }
  return MF_OK;
}

MF_EXPORT mf_status mf_bsr_upload(mf_ctx* ctx, mf_bsr* bsr, const int32_t* block_ptr_host,
                                  const int32_t* block_idx_host, const uint16_t* probs_host,
                                  const float* rkm_host) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  if (!block_ptr_host || !rkm_host) return fail(MF_ERR_INVALID, "block_ptr_host and row_kept_mass_host are required");
  const BsrOwner* own = static_cast<const BsrOwner*>(bsr->_owner);
  const Geometry& g = own->geom;
  if (block_ptr_host[0] != 0) return fail(MF_ERR_INVALID, "block_ptr[0] must be 0");
  for (int b = 0; b < g.n_brow; ++b)
    if (block_ptr_host[b + 1] < block_ptr_host[b]) return fail(MF_ERR_INVALID, "block_ptr decreases at row %d", b);
  const int64_t nnzb = block_ptr_host[g.n_brow];
  if (nnzb > bsr->capacity)
    return fail(MF_ERR_CAPACITY, "%lld blocks exceed the store capacity %lld", (long long)nnzb, (long long)bsr->capacity);
  if (nnzb > 0 && (!block_idx_host || !probs_host)) return fail(MF_ERR_INVALID, "block_idx_host / probs_host missing");
  std::vector<int32_t> rows((size_t)nnzb);
  for (int b = 0; b < g.n_brow; ++b) {
    const int I = g.info[4 * b + 3];
    for (int t = block_ptr_host[b]; t < block_ptr_host[b + 1]; ++t) {
      const int J = block_idx_host[t];
      if (J < 0 || J > I) return fail(MF_ERR_INVALID, "block column %d outside [0, %d] in row %d", J, I, b);
      if (t > block_ptr_host[b] && J <= block_idx_host[t - 1])
        return fail(MF_ERR_INVALID, "block columns of row %d are not ascending", b);
      rows[(size_t)t] = b;
    }
  }
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  MF_HIP(hipMemcpy(bsr->block_ptr, block_ptr_host, (size_t)(g.n_brow + 1) * 4, hipMemcpyHostToDevice), "copy block_ptr");
  if (nnzb > 0) {
    MF_HIP(hipMemcpy(bsr->block_idx, block_idx_host, (size_t)nnzb * 4, hipMemcpyHostToDevice), "copy block_idx");
    MF_HIP(hipMemcpy(bsr->block_row, rows.data(), (size_t)nnzb * 4, hipMemcpyHostToDevice), "copy block_row");
    MF_HIP(hipMemcpy(bsr->probs, probs_host, (size_t)nnzb * probs_block_bytes(bsr->H_s, bsr->B), hipMemcpyHostToDevice), "copy probs");
  }
  if (g.T) MF_HIP(hipMemcpy(bsr->row_kept_mass, rkm_host, (size_t)bsr->H_s * g.T * 4, hipMemcpyHostToDevice), "copy row_kept_mass");
  const int32_t cnt[2] = {(int32_t)nnzb, 0};
  MF_HIP(hipMemcpy(bsr->counters, cnt, sizeof(cnt), hipMemcpyHostToDevice), "copy counters");
  bsr->nnzb = nnzb;
  return MF_OK;
}

MF_EXPORT mf_status mf_compress_into(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype,
                                     int32_t d, float tau, mf_bsr* bsr, void* stream) {
  mf_status st = validate_compress(Q, K, dtype, d, tau, bsr);
  if (st != MF_OK) return st;
  if ((st = set_device(ctx)) != MF_OK) return st;
  if (bsr->n_brow == 0 || bsr->n_order == 0) return MF_OK;   // nothing to compress / retrieve
  hipStream_t s = static_cast<hipStream_t>(stream);
  mf::CompressArgs a;
  if ((st = prepare_compress_args(ctx, Q, K, dtype, d, tau, bsr, bsr->capacity, a, s)) != MF_OK) return st;
  MF_HIP(mf::compress_plan(a, s), "compress statistics / selection launch");
  MF_HIP(mf::compress_fill(a, s), "compress gather launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_compress_into_ex(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype,
                                        int32_t d, float tau, uint32_t options, mf_bsr* bsr, void* stream) {
  if (options & ~(uint32_t)(MF_SELECT_PER_HEAD | MF_NORM_PER_HEAD))
    return fail(MF_ERR_INVALID, "unknown option bits 0x%x", options);
  mf_status st = validate_compress(Q, K, dtype, d, tau, bsr);
  if (st != MF_OK) return st;
  if ((st = set_device(ctx)) != MF_OK) return st;
  if (bsr->n_brow == 0 || bsr->n_order == 0) return MF_OK;   // nothing to compress
  hipStream_t s = static_cast<hipStream_t>(stream);
  mf::CompressArgs a;
  if ((st = prepare_compress_args(ctx, Q, K, dtype, d, tau, bsr, bsr->capacity, a, s)) != MF_OK) return st;
  a.options = (int)options;
  if (options & MF_SELECT_PER_HEAD) {
    if ((st = ensure(ctx->al, ctx->hflags, (size_t)bsr->H_s * bsr->n_brow * bsr->nb_max + 256, "per-head flags", s)) != MF_OK)
      return st;
    a.hflags = static_cast<uint8_t*>(ctx->hflags.p);
  }
  if (options & MF_NORM_PER_HEAD) {
    if ((st = ensure(ctx->al, ctx->lse2n, (size_t)bsr->H_s * bsr->T * 4 + 256, "per-head logsumexp", s)) != MF_OK) return st;
    a.lse2n = static_cast<float*>(ctx->lse2n.p);
  }
  MF_HIP(mf::compress_plan(a, s), "compress statistics / selection launch");
  MF_HIP(mf::compress_fill(a, s), "compress gather launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_compress_prefill_into(mf_ctx* ctx, const void* Q, const void* K, const void* V,
                                             mf_dtype dtype, int32_t d, float tau, mf_bsr* bsr, float* O,
                                             void* stream) {
  mf_status st = validate_compress(Q, K, dtype, d, tau, bsr);
  if (st != MF_OK) return st;
  if (!V || !O) return fail(MF_ERR_INVALID, "V or O is NULL");
  if (!aligned16(V)) return fail(MF_ERR_INVALID, "V must be 16-byte aligned");
  if ((st = set_device(ctx)) != MF_OK) return st;
  if (bsr->n_brow == 0 || bsr->n_order == 0) return MF_OK;   // nothing to compress / retrieve
  hipStream_t s = static_cast<hipStream_t>(stream);
  const BsrOwner* bo = static_cast<const BsrOwner*>(bsr->_owner);
  st = vfrag_prepare(ctx, bo->geom.cu.data(), bsr->n_seq, bsr->B, V, dtype, bsr->H_s, d, nullptr, 0, 0,
                     &ctx->vf_prefill, true, s);
  if (st != MF_OK) return st;
  mf::CompressArgs a;
  if ((st = prepare_compress_args(ctx, Q, K, dtype, d, tau, bsr, bsr->capacity, a, s)) != MF_OK) return st;
  a.attn_vfrag = ctx->vf_prefill.frag;
  a.attn_vexps = ctx->vf_prefill.exps;
  a.attn_out = O;
  MF_HIP(mf::compress_plan(a, s), "fused prefill statistics / selection launch");
  MF_HIP(mf::compress_fill(a, s), "compress gather launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_bsr_sync(mf_ctx* ctx, mf_bsr* bsr, void* stream) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  int32_t cnt[2] = {0, 0};
  MF_HIP(hipMemcpy(cnt, bsr->counters, sizeof(cnt), hipMemcpyDeviceToHost), "reading kept-block count");
  bsr->nnzb = std::min<int64_t>(cnt[0], bsr->capacity);
  if (cnt[1]) return fail(MF_ERR_CAPACITY, "%d kept blocks exceed the store capacity %lld", cnt[0],
                          (long long)bsr->capacity);
  return MF_OK;
}

MF_EXPORT mf_status mf_compress(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype,
                                int32_t H_s, int32_t d, const int32_t* cu, int32_t n_seq, float tau,
                                int32_t B, void* stream, mf_bsr* out) {
  if (!out) return fail(MF_ERR_INVALID, "out is NULL");
  mf_bsr b{};
  mf_status st = mf_bsr_create(ctx, H_s, B, cu, n_seq, 0, &b);
  if (st != MF_OK) return st;
  if ((st = validate_compress(Q, K, dtype, d, tau, &b)) != MF_OK) {
    mf_bsr_free(ctx, &b);
    return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  BsrOwner* own = static_cast<BsrOwner*>(b._owner);
  if (b.n_brow > 0) {
    mf::CompressArgs a;
    // selection first with room for every causal block, then exact allocation
    if ((st = prepare_compress_args(ctx, Q, K, dtype, d, tau, &b, 0, a, s)) != MF_OK) {
      mf_bsr_free(ctx, &b);
      return st;
    }
    a.capacity = b.n_causal;
    hipError_t e = mf::compress_plan(a, s);
    if (e != hipSuccess) {
      mf_bsr_free(ctx, &b);
      return hip_fail(e, "compress statistics / selection launch");
    }
    int32_t cnt[2] = {0, 0};
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpy(cnt, b.counters, sizeof(cnt), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      mf_bsr_free(ctx, &b);
      return hip_fail(e, "reading kept-block count");
    }
    own->al.give(own->data, own->data_bytes, s);   // the stream is idle: nothing used the empty arrays
    own->data = nullptr;
    own->data_bytes = 0;
    if ((st = alloc_bsr_data(cnt[0], H_s, B, &b, own)) != MF_OK) {
      mf_bsr_free(ctx, &b);
      return st;
    }
    if ((st = prepare_compress_args(ctx, Q, K, dtype, d, tau, &b, b.capacity, a, s)) != MF_OK) {
      mf_bsr_free(ctx, &b);
      return st;
    }
    e = mf::compress_fill(a, s);
    if (e != hipSuccess) {
      mf_bsr_free(ctx, &b);
      return hip_fail(e, "compress gather launch");
    }
    b.nnzb = cnt[0];
  }
  *out = b;
  return MF_OK;
}

MF_EXPORT mf_status mf_v_prepare(mf_ctx* ctx, const int32_t* cu, int32_t n_seq, int32_t B,
                                 const void* V, mf_dtype dtype, int32_t H_kv, int32_t d,
                                 const int32_t* page_table, int32_t page_size,
                                 int32_t pages_per_seq, mf_vfrag* out, void* stream) {
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  if (out && out->_owner) {
    // re-preparation into the same buffers: the geometry must be unchanged
    const VfragOwner* own = static_cast<const VfragOwner*>(out->_owner);
    Geometry g;
    if ((st = build_geometry(cu, n_seq, B, g)) != MF_OK) return st;
    if (!(own->geom.cu == g.cu && own->geom.B == B && out->H_kv == H_kv && out->d == d))
      return fail(MF_ERR_INVALID, "prepared V exists with a different geometry; free it first");
  }
  return vfrag_prepare(ctx, cu, n_seq, B, V, dtype, H_kv, d, page_table, page_size, pages_per_seq,
                       out, out && out->_owner, static_cast<hipStream_t>(stream));
}

MF_EXPORT mf_status mf_vfrag_free(mf_ctx* ctx, mf_vfrag* vf) {
  if (ctx) (void)hipSetDevice(ctx->device);
  if (vf && vf->_owner) (void)hipDeviceSynchronize();   // no enqueued work may still use it
  vfrag_release(vf);
  return MF_OK;
}

// One launch for n_recv receivers of the same store: every receiver's head parts are splits of
// one row-tile work item, so each stored probability tile is read from HBM once for all of them.
// vf_from_store: the prepared V was laid out on the store's own geometry tables (it has no owner)
static mf_status retrieve_launch(mf_ctx* ctx, const mf_bsr* bsr, int n_recv, const float* const* W,
                                 const int32_t* H_r, const mf_vfrag* const* vf,
                                 const int32_t* const* kvmap, float* const* O, void* stream,
                                 int accumulate = 0, float* den = nullptr, bool vf_from_store = false) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  if (n_recv < 1 || n_recv > mf::kMaxRecv)
    return fail(MF_ERR_INVALID, "n_recv = %d outside [1, %d]", n_recv, mf::kMaxRecv);
  if (!W || !H_r || !vf || !kvmap || !O) return fail(MF_ERR_INVALID, "receiver array is NULL");
  const BsrOwner* bo = static_cast<const BsrOwner*>(bsr->_owner);
  mf::RetrieveArgs a{};
  mf::HeadMap hm[mf::kMaxRecv];
  for (int r = 0; r < n_recv; ++r) {
    const mf_vfrag* v = vf[r];
    if (!v || !(v->_owner || vf_from_store)) return fail(MF_ERR_INVALID, "prepared V of receiver %d is NULL", r);
    if (!W[r] || !O[r]) return fail(MF_ERR_INVALID, "W or O of receiver %d is NULL", r);
    if (H_r[r] < 1) return fail(MF_ERR_INVALID, "H_r of receiver %d must be >= 1", r);
    if (v->B != bsr->B || v->n_brow != bsr->n_brow || v->T != bsr->T)
      return fail(MF_ERR_INVALID, "prepared V of receiver %d: geometry (B=%d, %d block rows, T=%lld) "
                  "differs from the store's (B=%d, %d, T=%lld)", r, v->B, v->n_brow, (long long)v->T,
                  bsr->B, bsr->n_brow, (long long)bsr->T);
    const VfragOwner* vo = static_cast<const VfragOwner*>(v->_owner);
    if (!vf_from_store && vo->geom.cu != bo->geom.cu)
      return fail(MF_ERR_INVALID, "prepared V of receiver %d has different cu_seqlens", r);
    if (v->d != vf[0]->d)
      return fail(MF_ERR_INVALID, "receiver %d has head dim %d, receiver 0 has %d", r, v->d, vf[0]->d);
    if (!mf::retrieve_supported(bsr->B, v->d, H_r[r], bsr->H_s))
      return fail(MF_ERR_UNSUPPORTED, "no retrieve kernel for B=%d d=%d H_r=%d H_s=%d", bsr->B, v->d,
                  H_r[r], bsr->H_s);
    mf::RecvArgs& rv = a.recv[r];
    mf_status st = build_headmap(kvmap[r], H_r[r], v->H_kv, hm[r]);
    if (st != MF_OK) return st;
    rv.W = W[r];
    rv.vfrag = v->frag;
    rv.vexps = v->exps;
    rv.O = O[r];
    rv.H_r = H_r[r];
    rv.H_kv = v->H_kv;
    rv.den = den;
  }
  // Head splits.  Each receiver's heads (in KV order) form one part, or two equal parts above 24
  // heads.  Parts are packed first-fit, largest first, into splits of at most 24 heads (a split
  // may hold parts of several receivers).  A workgroup costs about the same per kept block
  // whatever its head count within one width, and the splits of one row tile only share the P
  // tile through L2 while they advance at the same rate, so splits are grouped by width
  // (HP = ceil(heads / 8)) and each group is one launch.
  // A grouped-query receiver of 32 heads whose KV groups fill whole waves (4 heads each, in KV
  // order) is the exception: it forms one 32-head part with a split of its own, run on the
  // half-block fast path (B = 64), so its P tiles are read once per row tile.
  bool whole32[mf::kMaxRecv];
  for (int r = 0; r < n_recv; ++r) {
    whole32[r] = H_r[r] == 32 && bsr->B == 64;
    for (int wv = 0; whole32[r] && wv < 8; ++wv)
      for (int i = 1; i < 4; ++i)
        if (hm[r].kv[hm[r].perm[4 * wv + i]] != hm[r].kv[hm[r].perm[4 * wv]]) whole32[r] = false;
  }
  struct Part { int r, g0, n; };
  Part parts[2 * mf::kMaxRecv];
  int n_parts = 0;
  for (int r = 0; r < n_recv; ++r) {
    const int halves = (H_r[r] <= mf::kSplitMax || whole32[r]) ? 1 : 2;
    for (int p = 0, g0 = 0; p < halves; ++p) {
      const int n = H_r[r] / halves + (p < H_r[r] % halves ? 1 : 0);
      parts[n_parts++] = Part{r, g0, n};
      g0 += n;
    }
  }
  std::stable_sort(parts, parts + n_parts, [](const Part& x, const Part& y) { return x.n > y.n; });
  int split_of[2 * mf::kMaxRecv], split_heads[2 * mf::kMaxRecv], n_split = 0;
  for (int i = 0; i < n_parts; ++i) {
    int k = 0;
    // a part above kSplitMax heads (a whole 32-head receiver) opens a split that nothing joins
    while (k < n_split && (split_heads[k] + parts[i].n > mf::kSplitMax)) ++k;
    if (k == n_split) split_heads[n_split++] = 0;
    split_heads[k] += parts[i].n;
    split_of[i] = k;
  }
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  if (bsr->n_brow == 0 || bsr->n_order == 0) return MF_OK;   // nothing to compress / retrieve
  a.probs = bsr->probs;
  a.block_ptr = bsr->block_ptr;
  a.block_idx = bsr->block_idx;
  a.info = bsr->brow_info;
  a.order = bsr->brow_order;
  a.capacity = bsr->capacity;
  a.n_brow = bsr->n_brow;
  a.n_order = bsr->n_order;
  a.H_s = bsr->H_s;
  a.B = bsr->B;
  a.d = vf[0]->d;
  a.T = bsr->T;
  a.rkm = bsr->row_kept_mass;
  a.n_recv = n_recv;
  a.accumulate = accumulate;
  for (int HP = 1; HP <= 4; ++HP) {
    a.HP = HP;
    a.n_split = 0;
    for (int k = 0; k < n_split; ++k) {
      if ((split_heads[k] + 7) / 8 != HP) continue;
      const int ks = a.n_split++;
      int j = 0;
      for (int i = 0; i < n_parts; ++i) {
        if (split_of[i] != k) continue;
        const Part& pt = parts[i];
        for (int q = 0; q < pt.n; ++q, ++j) {
          const int head = hm[pt.r].perm[pt.g0 + q];
          a.slot_recv[ks][j] = (int8_t)pt.r;
          a.slot_head[ks][j] = (int8_t)head;
          a.slot_kv[ks][j] = hm[pt.r].kv[head];
        }
      }
      a.split_nslots[ks] = (int8_t)j;
      for (; j < mf::kMaxSlots; ++j) {
        a.slot_recv[ks][j] = 0;
        a.slot_head[ks][j] = -1;
        a.slot_kv[ks][j] = 0;
      }
    }
    if (a.n_split == 0) continue;
    MF_HIP(mf::retrieve(a, static_cast<hipStream_t>(stream)), "retrieve launch");
  }
  return MF_OK;
}

MF_EXPORT mf_status mf_retrieve_prepared(mf_ctx* ctx, const mf_bsr* bsr, const float* W,
                                         int32_t H_r, const mf_vfrag* vf,
                                         const int32_t* kvmap, float* O, void* stream) {
  if (!W || !O) return fail(MF_ERR_INVALID, "W or O is NULL");
  if (!vf || !vf->_owner) return fail(MF_ERR_INVALID, "prepared V is NULL");
  return retrieve_launch(ctx, bsr, 1, &W, &H_r, &vf, &kvmap, &O, stream);
}

MF_EXPORT mf_status mf_retrieve_multi(mf_ctx* ctx, const mf_bsr* bsr, int32_t n_recv,
                                      const float* const* W, const int32_t* H_r,
                                      const mf_vfrag* const* vf, const int32_t* const* kvmap,
                                      float* const* O, void* stream) {
  return retrieve_launch(ctx, bsr, n_recv, W, H_r, vf, kvmap, O, stream);
}

MF_EXPORT mf_status mf_retrieve_layers(mf_ctx* ctx, int32_t n_layers, const mf_bsr* stores,
                                       const float* const* W, int32_t H_r, const mf_vfrag* vf,
                                       const int32_t* kvmap, float* O, void* stream) {
  if (n_layers < 1 || !stores || !W) return fail(MF_ERR_INVALID, "need n_layers >= 1 stores and weights");
  if (n_layers == 1) return mf_retrieve_prepared(ctx, &stores[0], W[0], H_r, vf, kvmap, O, stream);
  for (int l = 0; l < n_layers; ++l) {
    const mf_bsr& b = stores[l];
    if (!b._owner || !W[l]) return fail(MF_ERR_INVALID, "store or W of layer %d is NULL", l);
    const BsrOwner* o0 = static_cast<const BsrOwner*>(stores[0]._owner);
    const BsrOwner* ol = static_cast<const BsrOwner*>(b._owner);
    if (b.B != stores[0].B || ol->geom.cu != o0->geom.cu || ol->geom.active != o0->geom.active)
      return fail(MF_ERR_INVALID, "store of layer %d has another geometry (B, cu_seqlens or row range)", l);
  }
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  if ((st = ensure(ctx->al, ctx->den, (size_t)stores[0].T * H_r * 4 + 256, "denominators", static_cast<hipStream_t>(stream))) != MF_OK) return st;
  float* den = static_cast<float*>(ctx->den.p);
  for (int l = 0; l < n_layers; ++l) {
    const int mode = l == 0 ? 1 : (l + 1 < n_layers ? 2 : 3);
    const float* Wl = W[l];
    st = retrieve_launch(ctx, &stores[l], 1, &Wl, &H_r, &vf, &kvmap, &O, stream, mode, den);
    if (st != MF_OK) return st;
  }
  return MF_OK;
}

MF_EXPORT mf_status mf_retrieve(mf_ctx* ctx, const mf_bsr* bsr, const float* W, int32_t H_r,
                                const void* V, mf_dtype vdtype, int32_t H_kv, int32_t d,
                                const int32_t* page_table, int32_t page_size, int32_t pages_per_seq,
                                const int32_t* kvmap, float* O, void* stream) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  const BsrOwner* bo = static_cast<const BsrOwner*>(bsr->_owner);
  if (!mf::retrieve_supported(bsr->B, d, H_r, bsr->H_s))
    return fail(MF_ERR_UNSUPPORTED, "no retrieve kernel for B=%d d=%d H_r=%d H_s=%d", bsr->B, d, H_r, bsr->H_s);
  mf::HeadMap hm;
  if ((st = build_headmap(kvmap, H_r, H_kv, hm)) != MF_OK) return st;
  if (!W || !O) return fail(MF_ERR_INVALID, "W or O is NULL");
  st = vfrag_prepare(ctx, bo->geom.cu.data(), bsr->n_seq, bsr->B, V, vdtype, H_kv, d, page_table,
                     page_size, pages_per_seq, &ctx->vf_retrieve, true, static_cast<hipStream_t>(stream));
  if (st != MF_OK) return st;
  return mf_retrieve_prepared(ctx, bsr, W, H_r, &ctx->vf_retrieve, kvmap, O, stream);
}

MF_EXPORT mf_status mf_dense_attention(mf_ctx* ctx, const void* Q, const void* K, const void* V,
                                       mf_dtype dtype, int32_t H_q, int32_t H_kv, int32_t d,
                                       const int32_t* cu, int32_t n_seq, const int32_t* kvmap,
                                       float* O, void* stream) {
  if (!Q || !K || !V || !O) return fail(MF_ERR_INVALID, "Q, K, V or O is NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V))
    return fail(MF_ERR_INVALID, "Q, K and V must be 16-byte aligned");
  mf_status st = check_dtype(dtype);
  if (st != MF_OK) return st;
  if (!mf::dense_supported(dtype_code(dtype), d))
    return fail(MF_ERR_UNSUPPORTED, "dense attention supports d = 64 or 128 (got %d)", d);
  if (H_kv < 1 || H_kv > 64) return fail(MF_ERR_INVALID, "H_kv must be in [1, 64]");
  mf::HeadMap hm;
  if ((st = build_headmap(kvmap, H_q, H_kv, hm)) != MF_OK) return st;
  Geometry g;
  if ((st = build_geometry(cu, n_seq, 64, g)) != MF_OK) return st;
  if ((st = set_device(ctx)) != MF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.n_brow == 0) return MF_OK;
  // geometry tables (info, order) cached on the device while cu_seqlens stays the same
  if (ctx->dense_cu != g.cu) {
    const size_t o_order = align_up((size_t)g.n_brow * 16, 256);
    const size_t o_pairs = align_up(o_order + (size_t)g.n_brow * 4, 256);
    if ((st = ensure(ctx->al, ctx->dense_tables, o_pairs + (size_t)g.n_pair * 8 + 256, "dense geometry", s)) != MF_OK) return st;
    char* base = static_cast<char*>(ctx->dense_tables.p);
    MF_HIP(hipMemcpy(base, g.info.data(), (size_t)g.n_brow * 16, hipMemcpyHostToDevice), "uploading geometry");
    MF_HIP(hipMemcpy(base + o_order, g.order.data(), (size_t)g.n_order * 4, hipMemcpyHostToDevice),
           "uploading geometry");
    MF_HIP(hipMemcpy(base + o_pairs, g.pairs.data(), (size_t)g.n_pair * 8, hipMemcpyHostToDevice),
           "uploading geometry");
    ctx->dense_cu = g.cu;
    ctx->dense_nbrow = g.n_brow;
  }
  st = vfrag_prepare(ctx, cu, n_seq, 64, V, dtype, H_kv, d, nullptr, 0, 0, &ctx->vf_dense, true, s);
  if (st != MF_OK) return st;
  char* base = static_cast<char*>(ctx->dense_tables.p);
  mf::DenseArgs a{};
  a.Q = Q;
  a.K = K;
  a.dtype = dtype_code(dtype);
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.d = d;
  a.T = g.T;
  a.n_brow = g.n_brow;
  a.info = reinterpret_cast<const int32_t*>(base);
  a.order = reinterpret_cast<const int32_t*>(base + align_up((size_t)g.n_brow * 16, 256));
  a.pairs = reinterpret_cast<const int32_t*>(
      base + align_up(align_up((size_t)g.n_brow * 16, 256) + (size_t)g.n_brow * 4, 256));
  a.n_pair = g.n_pair;
  a.vfrag = ctx->vf_dense.frag;
  a.vexps = ctx->vf_dense.exps;
  a.hm = hm;
  a.O = O;
  MF_HIP(mf::dense_attention(a, s), "dense attention launch");
  return MF_OK;
}

// ------------------------------------------------------------------------------------------
// Receiver prefill over every layer: dense recompute of the first R layers and the fused retrieve
// of the mapped ones, with the compress of later layers' sender maps on a second stream.
// ------------------------------------------------------------------------------------------

MF_EXPORT mf_status mf_prefill_layers(mf_ctx* ctx, const mf_recv_layer* recv, const mf_send_layer* send,
                                      mf_dtype dtype, int32_t H_r, int32_t H_kv, int32_t d,
                                      const int32_t* kvmap, float tau, int32_t n_slots, mf_bsr* slots,
                                      uint32_t flags, void* stream_main, void* stream_prefetch) {
  if (!ctx) return fail(MF_ERR_INVALID, "context is NULL");
  if (ctx->pi.empty()) return fail(MF_ERR_INVALID, "no layer map installed: call mf_map_layers first");
  if (!recv || !send) return fail(MF_ERR_INVALID, "recv or send is NULL");
  if (flags & ~(uint32_t)(MF_PREFILL_ISOLATE | MF_PREFILL_TIMING))
    return fail(MF_ERR_INVALID, "unknown flag bits 0x%x", flags);
  if (n_slots < 1 || !slots) return fail(MF_ERR_INVALID, "need n_slots >= 1 stores (got %d)", n_slots);
  mf_status st = check_dtype(dtype);
  if (st != MF_OK) return st;
  if (!(tau > 0.f && tau <= 1.f)) return fail(MF_ERR_INVALID, "tau must be in (0, 1] (got %g)", (double)tau);
  if (d != 64 && d != 128) return fail(MF_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
  if (H_kv < 1 || H_kv > 64) return fail(MF_ERR_INVALID, "H_kv must be in [1, 64] (got %d)", H_kv);
  mf::HeadMap hm;
  if ((st = build_headmap(kvmap, H_r, H_kv, hm)) != MF_OK) return st;

  // the ring: stores of one geometry, each able to hold every causal block
  const BsrOwner* o0 = static_cast<const BsrOwner*>(slots[0]._owner);
  if (!o0) return fail(MF_ERR_INVALID, "slot 0 is not a block store");
  for (int i = 0; i < n_slots; ++i) {
    const mf_bsr& b = slots[i];
    const BsrOwner* o = static_cast<const BsrOwner*>(b._owner);
    if (!o) return fail(MF_ERR_INVALID, "slot %d is not a block store", i);
    if (o->cache_owned) return fail(MF_ERR_INVALID, "slot %d is a prefix-cache view (read-only)", i);
    if (o->geom.ranged) return fail(MF_ERR_INVALID, "slot %d is a row-range store", i);
    if (b.B != slots[0].B || b.H_s != slots[0].H_s || o->geom.cu != o0->geom.cu)
      return fail(MF_ERR_INVALID, "slot %d has another geometry than slot 0 (B, H_s or cu_seqlens)", i);
    if (b.capacity < b.n_causal)
      return fail(MF_ERR_INVALID, "slot %d holds %lld blocks, fewer than its %lld causal blocks", i,
                  (long long)b.capacity, (long long)b.n_causal);
    for (int j = 0; j < i; ++j)
      if (slots[j].probs == b.probs) return fail(MF_ERR_INVALID, "slots %d and %d are the same store", j, i);
  }
  const int B = slots[0].B, H_s = slots[0].H_s;
  if (!mf::retrieve_supported(B, d, H_r, H_s))
    return fail(MF_ERR_UNSUPPORTED, "no retrieve kernel for B=%d d=%d H_r=%d H_s=%d", B, d, H_r, H_s);
  const int n_recv = ctx->n_recv, R = ctx->R;
  const std::vector<int32_t> pi = ctx->pi;
  std::vector<int> mapped;
  for (int l = 0; l < n_recv; ++l)
    if (pi[l] >= 0) mapped.push_back(l);
  const int n_map = (int)mapped.size();
  for (int l = 0; l < n_recv; ++l) {
    const mf_recv_layer& r = recv[l];
    if (!r.V || !r.O) return fail(MF_ERR_INVALID, "receiver layer %d: V or O is NULL", l);
    if (!aligned16(r.V)) return fail(MF_ERR_INVALID, "receiver layer %d: V must be 16-byte aligned", l);
    if (pi[l] < 0) {
      if (!r.Q || !r.K) return fail(MF_ERR_INVALID, "recomputed receiver layer %d: Q or K is NULL", l);
      if (!aligned16(r.Q) || !aligned16(r.K))
        return fail(MF_ERR_INVALID, "recomputed receiver layer %d: Q and K must be 16-byte aligned", l);
    } else {
      if (!r.W) return fail(MF_ERR_INVALID, "mapped receiver layer %d: W is NULL", l);
      if ((st = validate_compress(send[pi[l]].Q, send[pi[l]].K, dtype, d, tau, &slots[0])) != MF_OK) return st;
    }
  }
  if (R > 0 && !mf::dense_supported(dtype_code(dtype), d))
    return fail(MF_ERR_UNSUPPORTED, "dense attention supports d = 64 or 128 (got %d)", d);
  if ((st = set_device(ctx)) != MF_OK) return st;

  // events: start, end, then per layer
  PrefillState& P = ctx->pre;
  const bool timing = (flags & MF_PREFILL_TIMING) != 0, isolate = (flags & MF_PREFILL_ISOLATE) != 0;
  int n_ev = 0;
  auto take = [&n_ev](std::vector<int>& v, int n) {
    v.resize(n);
    for (int i = 0; i < n; ++i) v[i] = n_ev++;
  };
  P.e_start = n_ev++;
  P.e_end = n_ev++;
  take(P.d0, R);
  take(P.d1, R);
  take(P.c0, n_map);
  take(P.c1, n_map);
  take(P.v0, n_map);
  take(P.r0, n_map);
  take(P.r1, n_map);
  while ((int)P.ev.size() < n_ev) {
    hipEvent_t e;
    MF_HIP(hipEventCreate(&e), "hipEventCreate");
    P.ev.push_back(e);
  }
  P.timed = false;
  P.n_map = n_map;
  P.R = R;
  auto E = [&P](int i) { return P.ev[i]; };
  hipStream_t sa = static_cast<hipStream_t>(stream_main), sb = static_cast<hipStream_t>(stream_prefetch);
  const int32_t* cu = o0->geom.cu.data();
  const int n_seq = slots[0].n_seq;

  // both streams start after the caller's earlier work on stream_main
  MF_HIP(hipEventRecord(E(P.e_start), sa), "hipEventRecord");
  MF_HIP(hipStreamWaitEvent(sb, E(P.e_start), 0), "hipStreamWaitEvent");

  // compress of the m-th mapped layer into slot m % n_slots, once the retrieve that last read the
  // slot has finished
  auto compress = [&](int m) -> mf_status {
    if (m >= n_slots) MF_HIP(hipStreamWaitEvent(sb, E(P.r1[m - n_slots]), 0), "hipStreamWaitEvent");
    if (timing) MF_HIP(hipEventRecord(E(P.c0[m]), sb), "hipEventRecord");
    const mf_send_layer& sl = send[pi[mapped[m]]];
    const mf_status cs = mf_compress_into(ctx, sl.Q, sl.K, dtype, d, tau, &slots[m % n_slots], sb);
    if (cs != MF_OK) return cs;
    MF_HIP(hipEventRecord(E(P.c1[m]), sb), "hipEventRecord");
    return MF_OK;
  };
  int enq = 0;   // compresses enqueued so far
  for (; enq < std::min(n_slots, n_map); ++enq)
    if ((st = compress(enq)) != MF_OK) return st;
  // stream_main recomputes the first R layers meanwhile
  for (int l = 0; l < R; ++l) {
    const mf_recv_layer& r = recv[l];
    if (timing) MF_HIP(hipEventRecord(E(P.d0[l]), sa), "hipEventRecord");
    if ((st = mf_dense_attention(ctx, r.Q, r.K, r.V, dtype, H_r, H_kv, d, cu, n_seq, kvmap, r.O, sa)) != MF_OK)
      return st;
    if (timing) MF_HIP(hipEventRecord(E(P.d1[l]), sa), "hipEventRecord");
  }
  for (int m = 0; m < n_map; ++m) {
    const mf_recv_layer& r = recv[mapped[m]];
    // isolated: wait for the last compress enqueued so far (the prefetch stream is then idle);
    // overlapped: wait for this slot's compress only
    MF_HIP(hipStreamWaitEvent(sa, E(P.c1[isolate ? enq - 1 : m]), 0), "hipStreamWaitEvent");
    if (timing) MF_HIP(hipEventRecord(E(P.v0[m]), sa), "hipEventRecord");
    if ((st = vfrag_prepare(ctx, cu, n_seq, B, r.V, dtype, H_kv, d, nullptr, 0, 0, &ctx->vf_pipe, true, sa)) != MF_OK)
      return st;
    if (timing) MF_HIP(hipEventRecord(E(P.r0[m]), sa), "hipEventRecord");
    const mf_vfrag* vfp = &ctx->vf_pipe;
    const float* W = r.W;
    float* O = r.O;
    if ((st = retrieve_launch(ctx, &slots[m % n_slots], 1, &W, &H_r, &vfp, &kvmap, &O, sa)) != MF_OK) return st;
    MF_HIP(hipEventRecord(E(P.r1[m]), sa), "hipEventRecord");
    if (enq < n_map) {
      if ((st = compress(enq)) != MF_OK) return st;
      ++enq;
    }
  }
  // stream_main's later work follows the last compress as well
  MF_HIP(hipEventRecord(E(P.e_end), sb), "hipEventRecord");
  MF_HIP(hipStreamWaitEvent(sa, E(P.e_end), 0), "hipStreamWaitEvent");
  P.timed = timing;
  return MF_OK;
}

MF_EXPORT mf_status mf_prefill_timings(mf_ctx* ctx, float* dense_ms, float* compress_ms, float* vprep_ms,
                                       float* retrieve_ms) {
  if (!ctx) return fail(MF_ERR_INVALID, "context is NULL");
  const PrefillState& P = ctx->pre;
  if (!P.timed) return fail(MF_ERR_INVALID, "the last mf_prefill_layers call recorded no timing events");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  auto span = [&P](int a, int b, float* out) -> mf_status {
    MF_HIP(hipEventSynchronize(P.ev[b]), "hipEventSynchronize");
    MF_HIP(hipEventElapsedTime(out, P.ev[a], P.ev[b]), "hipEventElapsedTime");
    return MF_OK;
  };
  for (int l = 0; l < P.R && dense_ms; ++l)
    if ((st = span(P.d0[l], P.d1[l], &dense_ms[l])) != MF_OK) return st;
  for (int m = 0; m < P.n_map; ++m) {
    if (compress_ms && (st = span(P.c0[m], P.c1[m], &compress_ms[m])) != MF_OK) return st;
    if (vprep_ms && (st = span(P.v0[m], P.r0[m], &vprep_ms[m])) != MF_OK) return st;
    if (retrieve_ms && (st = span(P.r0[m], P.r1[m], &retrieve_ms[m])) != MF_OK) return st;
  }
  return MF_OK;
}

// ------------------------------------------------------------------------------------------
// Prefix-hash cache of compressed block rows.
// ------------------------------------------------------------------------------------------

namespace {

// FNV-1a, 64-bit (offset basis 0xcbf29ce484222325, prime 0x100000001b3), over little-endian bytes.
uint64_t fnv1a64(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

void prefix_hashes(const int32_t* tokens, int64_t n_rows, int32_t B, uint64_t* out) {
  uint64_t h = fnv1a64(0xcbf29ce484222325ull, &B, 4);
  for (int64_t r = 0; r < n_rows; ++r) {
    h = fnv1a64(0xcbf29ce484222325ull, &h, 8);
    h = fnv1a64(h, tokens + r * B, (size_t)B * 4);
    out[r] = h;
  }
}

struct CacheKey {
  int32_t layer, rows;
  uint64_t hash;
  bool operator==(const CacheKey& o) const { return layer == o.layer && rows == o.rows && hash == o.hash; }
};
struct CacheKeyHash {
  size_t operator()(const CacheKey& k) const {
    return (size_t)(k.hash ^ ((uint64_t)(uint32_t)k.layer << 32) ^ (uint64_t)(uint32_t)k.rows * 0x9e3779b97f4a7c15ull);
  }
};

struct CacheEntry {
  mf_bsr bsr{};                   // single sequence of rows * B tokens, every row compressed
  std::vector<int32_t> tokens;    // the prefix, to confirm a hash match
  size_t bytes = 0;
  uint64_t last_use = 0;
};

}  // namespace

struct mf_cache {
  mf_ctx* ctx = nullptr;
  int64_t budget = 0, used = 0;
  uint64_t clock = 0;
  std::unordered_map<CacheKey, std::unique_ptr<CacheEntry>, CacheKeyHash> map;
};

namespace {

void cache_drop(mf_cache* c, std::unordered_map<CacheKey, std::unique_ptr<CacheEntry>, CacheKeyHash>::iterator it) {
  CacheEntry* e = it->second.get();
  BsrOwner* own = static_cast<BsrOwner*>(e->bsr._owner);
  if (own) {
    own->cache_owned = false;
    mf_bsr_free(c->ctx, &e->bsr);
  }
  c->used -= (int64_t)e->bytes;
  c->map.erase(it);
}

}  // namespace

MF_EXPORT mf_status mf_prefix_hashes(const int32_t* tokens, int64_t n_tokens, int32_t B, uint64_t* out) {
  if (n_tokens < 0) return fail(MF_ERR_INVALID, "n_tokens must be >= 0");
  if (B < 1) return fail(MF_ERR_INVALID, "B must be >= 1");
  if (n_tokens / B > 0 && (!tokens || !out)) return fail(MF_ERR_INVALID, "tokens or hashes_out is NULL");
  prefix_hashes(tokens, n_tokens / B, B, out);
  return MF_OK;
}

MF_EXPORT mf_status mf_cache_create(mf_ctx* ctx, int64_t budget_bytes, mf_cache** out) {
  if (!ctx) return fail(MF_ERR_INVALID, "context is NULL");
  if (!out) return fail(MF_ERR_INVALID, "out is NULL");
  if (budget_bytes <= 0) return fail(MF_ERR_INVALID, "budget_bytes must be > 0");
  mf_cache* c = new (std::nothrow) mf_cache();
  if (!c) return fail(MF_ERR_OOM, "host allocation failed");
  c->ctx = ctx;
  c->budget = budget_bytes;
  *out = c;
  return MF_OK;
}

MF_EXPORT mf_status mf_cache_destroy(mf_cache* cache) {
  if (!cache) return MF_OK;
  if (cache->ctx) (void)hipSetDevice(cache->ctx->device);
  (void)hipDeviceSynchronize();
  while (!cache->map.empty()) cache_drop(cache, cache->map.begin());
  delete cache;
  return MF_OK;
}

MF_EXPORT mf_status mf_cache_info(const mf_cache* cache, int64_t* entries, int64_t* used_bytes) {
  if (!cache) return fail(MF_ERR_INVALID, "cache is NULL");
  if (entries) *entries = (int64_t)cache->map.size();
  if (used_bytes) *used_bytes = cache->used;
  return MF_OK;
}

MF_EXPORT mf_status mf_cache_insert(mf_cache* cache, int32_t layer, const int32_t* tokens, int64_t n_tokens,
                                    int32_t n_parts, const mf_bsr* parts, int32_t rows, void* stream) {
  if (!cache) return fail(MF_ERR_INVALID, "cache is NULL");
  if (n_parts < 1 || !parts) return fail(MF_ERR_INVALID, "need at least one part store");
  const int B = parts[0].B, H_s = parts[0].H_s;
  if (rows < 1 || (int64_t)rows * B > n_tokens)
    return fail(MF_ERR_INVALID, "rows = %d must be in [1, n_tokens / B = %lld]", rows, (long long)(n_tokens / B));
  if (!tokens) return fail(MF_ERR_INVALID, "tokens is NULL");
  // every row 0..rows-1 comes from the first part that compresses it
  std::vector<int> src(rows, -1);
  for (int k = 0; k < n_parts; ++k) {
    const mf_bsr& p = parts[k];
    const BsrOwner* po = static_cast<const BsrOwner*>(p._owner);
    if (!po) return fail(MF_ERR_INVALID, "part %d is not a store", k);
    if (p.n_seq != 1) return fail(MF_ERR_INVALID, "part %d holds %d sequences; parts are single sequences", k, p.n_seq);
    if (p.B != B || p.H_s != H_s) return fail(MF_ERR_INVALID, "part %d has B = %d, H_s = %d; part 0 has %d, %d", k, p.B, p.H_s, B, H_s);
    for (int r = 0; r < rows && r < p.n_brow; ++r) {
      // a row's content depends on its full block of queries: only rows complete in the part count
      if (src[r] < 0 && po->geom.active[r] && (int64_t)(r + 1) * B <= p.T) src[r] = k;
    }
  }
  for (int r = 0; r < rows; ++r)
    if (src[r] < 0) return fail(MF_ERR_INVALID, "block row %d is compressed (complete) in none of the parts", r);
  mf_status st = set_device(cache->ctx);
  if (st != MF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // block counts per row from the parts' block_ptr
  std::vector<std::vector<int32_t>> ptrs(n_parts);
  for (int k = 0; k < n_parts; ++k) {
    ptrs[k].resize((size_t)parts[k].n_brow + 1);
    MF_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");
    MF_HIP(hipMemcpy(ptrs[k].data(), parts[k].block_ptr, ptrs[k].size() * 4, hipMemcpyDeviceToHost), "reading block_ptr");
  }
  std::vector<int32_t> new_ptr(rows + 1, 0);
  for (int r = 0; r < rows; ++r) new_ptr[r + 1] = new_ptr[r] + ptrs[src[r]][r + 1] - ptrs[src[r]][r];
  const int64_t nnzb = new_ptr[rows];
  const size_t bytes = (size_t)nnzb * (8 + probs_block_bytes(H_s, B)) + (size_t)H_s * rows * B * 4 + (size_t)rows * 64;
  if ((int64_t)bytes > cache->budget)
    return fail(MF_ERR_CAPACITY, "entry of %zu bytes exceeds the cache budget %lld", bytes, (long long)cache->budget);
  uint64_t h_last = 0;
  {
    std::vector<uint64_t> hs(rows);
    prefix_hashes(tokens, rows, B, hs.data());
    h_last = hs[rows - 1];
  }
  const CacheKey key{layer, rows, h_last};
  auto found = cache->map.find(key);
  if (found != cache->map.end() && std::equal(found->second->tokens.begin(), found->second->tokens.end(), tokens)) {
    found->second->last_use = ++cache->clock;       // already cached
    return MF_OK;
  }
  if (found != cache->map.end()) cache_drop(cache, found);   // a colliding prefix: replace it
  while (cache->used + (int64_t)bytes > cache->budget && !cache->map.empty()) {
    auto lru = cache->map.begin();
    for (auto it = cache->map.begin(); it != cache->map.end(); ++it)
      if (it->second->last_use < lru->second->last_use) lru = it;
    cache_drop(cache, lru);
  }
  auto e = std::make_unique<CacheEntry>();
  const int32_t cu[2] = {0, rows * B};
  if ((st = bsr_create(cache->ctx, H_s, B, cu, 1, nullptr, nnzb, &e->bsr)) != MF_OK) return st;
  mf_bsr& d = e->bsr;
  MF_HIP(hipMemcpyAsync(d.block_ptr, new_ptr.data(), (size_t)(rows + 1) * 4, hipMemcpyHostToDevice, s), "copy block_ptr");
  const size_t pb = probs_block_bytes(H_s, B);
  for (int r = 0; r < rows;) {
    // one copy per run of rows from the same part
    int r1 = r + 1;
    while (r1 < rows && src[r1] == src[r]) ++r1;
    const mf_bsr& p = parts[src[r]];
    const int64_t a0 = ptrs[src[r]][r], a1 = ptrs[src[r]][r1], n = a1 - a0;
    if (n > 0) {
      MF_HIP(hipMemcpyAsync(d.block_idx + new_ptr[r], p.block_idx + a0, (size_t)n * 4, hipMemcpyDeviceToDevice, s), "copy block_idx");
      MF_HIP(hipMemcpyAsync(d.block_row + new_ptr[r], p.block_row + a0, (size_t)n * 4, hipMemcpyDeviceToDevice, s), "copy block_row");
      MF_HIP(hipMemcpyAsync(reinterpret_cast<char*>(d.probs) + (size_t)new_ptr[r] * pb,
                            reinterpret_cast<const char*>(p.probs) + (size_t)a0 * pb, (size_t)n * pb,
                            hipMemcpyDeviceToDevice, s), "copy probs");
    }
    MF_HIP(hipMemcpy2DAsync(d.row_kept_mass + (size_t)r * B, (size_t)rows * B * 4, p.row_kept_mass + (size_t)r * B,
                            (size_t)p.T * 4, (size_t)(r1 - r) * B * 4, H_s, hipMemcpyDeviceToDevice, s), "copy kept mass");
    r = r1;
  }
  const int32_t cnt[2] = {(int32_t)nnzb, 0};
  MF_HIP(hipMemcpyAsync(d.counters, cnt, sizeof(cnt), hipMemcpyHostToDevice, s), "copy counters");
  MF_HIP(hipStreamSynchronize(s), "hipStreamSynchronize");   // host sources above are stack / vector memory
  d.nnzb = nnzb;
  static_cast<BsrOwner*>(d._owner)->cache_owned = true;
  e->tokens.assign(tokens, tokens + (size_t)rows * B);
  e->bytes = bytes;
  e->last_use = ++cache->clock;
  cache->used += (int64_t)bytes;
  cache->map.emplace(key, std::move(e));
  return MF_OK;
}

MF_EXPORT mf_status mf_cache_lookup(mf_cache* cache, int32_t layer, const int32_t* tokens, int64_t n_tokens,
                                    int32_t B, int32_t* rows_out, mf_bsr* view_out) {
  if (!cache) return fail(MF_ERR_INVALID, "cache is NULL");
  if (!rows_out || !view_out) return fail(MF_ERR_INVALID, "rows_out or view_out is NULL");
  if (B < 1 || n_tokens < 0) return fail(MF_ERR_INVALID, "bad B or n_tokens");
  *rows_out = 0;
  std::memset(view_out, 0, sizeof(*view_out));
  const int64_t full = n_tokens / B;
  if (full == 0 || cache->map.empty()) return MF_OK;
  if (!tokens) return fail(MF_ERR_INVALID, "tokens is NULL");
  std::vector<uint64_t> hs((size_t)full);
  prefix_hashes(tokens, full, B, hs.data());
  for (int64_t r = full; r >= 1; --r) {
    auto it = cache->map.find(CacheKey{layer, (int32_t)r, hs[(size_t)r - 1]});
    if (it == cache->map.end() || it->second->bsr.B != B) continue;
    if (!std::equal(it->second->tokens.begin(), it->second->tokens.end(), tokens)) continue;
    it->second->last_use = ++cache->clock;
    *rows_out = (int32_t)r;
    *view_out = it->second->bsr;
    return MF_OK;
  }
  return MF_OK;
}

// ------------------------------------------------------------------------------------------
// Retrieve without any device allocation: the prepared V lives in a fixed device array.
// ------------------------------------------------------------------------------------------

}  // extern "C"

namespace {

// Prepared-V tiles (up to kNoAllocFragBytes) followed by the per-KV-head exponents and maxima.
constexpr size_t kNoAllocFragBytes = size_t(64) << 20;
constexpr size_t kNoAllocBytes = kNoAllocFragBytes + 4096;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

// Device address of `scratch` on each device, looked up once per device.  In host code the
// array's name is only a stand-in for the symbol; kernels get this address instead.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

mf_status scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return fail(MF_ERR_UNSUPPORTED, "device %d beyond %d", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[device]) {
    void* p = nullptr;
    MF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    g_scratch_addr[device] = p;
  }
  *out = g_scratch_addr[device];
  return MF_OK;
}

}  // namespace

extern "C" {

MF_EXPORT mf_status mf_retrieve_noalloc(mf_ctx* ctx, const mf_bsr* bsr, const float* W, int32_t H_r,
                                        const void* V, mf_dtype vdtype, int32_t H_kv, int32_t d,
                                        const int32_t* page_table, int32_t page_size, int32_t pages_per_seq,
                                        const int32_t* kvmap, float* O, void* stream) {
  if (!bsr || !bsr->_owner) return fail(MF_ERR_INVALID, "block store is NULL");
  if (!W || !O) return fail(MF_ERR_INVALID, "W or O is NULL");
  if (!V) return fail(MF_ERR_INVALID, "V is NULL");
  if (!aligned16(V)) return fail(MF_ERR_INVALID, "V must be 16-byte aligned");
  mf_status st = check_dtype(vdtype);
  if (st != MF_OK) return st;
  if (d != 64 && d != 128) return fail(MF_ERR_UNSUPPORTED, "head dim d must be 64 or 128 (got %d)", d);
  if (H_kv < 1 || H_kv > 64) return fail(MF_ERR_INVALID, "H_kv must be in [1, 64] (got %d)", H_kv);
  if (!mf::retrieve_supported(bsr->B, d, H_r, bsr->H_s))
    return fail(MF_ERR_UNSUPPORTED, "no retrieve kernel for B=%d d=%d H_r=%d H_s=%d", bsr->B, d, H_r, bsr->H_s);
  mf::HeadMap hm;
  if ((st = build_headmap(kvmap, H_r, H_kv, hm)) != MF_OK) return st;
  const BsrOwner* bo = static_cast<const BsrOwner*>(bsr->_owner);
  const Geometry& g = bo->geom;
  if (page_table) {
    if (page_size < 1 || pages_per_seq < 1)
      return fail(MF_ERR_INVALID, "paged V needs page_size >= 1 and pages_per_seq >= 1");
    for (int s = 0; s < bsr->n_seq; ++s)
      if ((int64_t)(g.cu[s + 1] - g.cu[s]) > (int64_t)page_size * pages_per_seq)
        return fail(MF_ERR_INVALID, "sequence %d needs more than pages_per_seq pages", s);
  }
  const size_t frag_bytes = (size_t)H_kv * bsr->n_brow * bsr->B * d * 2;
  if (frag_bytes > kNoAllocFragBytes)
    return fail(MF_ERR_UNSUPPORTED, "prepared V needs %zu bytes, more than the %zu-byte fixed scratch "
                "(H_kv x block rows x B x d fp16 values)", frag_bytes, kNoAllocFragBytes);
  if ((st = set_device(ctx)) != MF_OK) return st;
  if (bsr->n_brow == 0 || bsr->n_order == 0) return MF_OK;
  void* base = nullptr;
  if ((st = scratch_address(ctx->device, &base)) != MF_OK) return st;
  unsigned char* p = static_cast<unsigned char*>(base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  mf_vfrag vf{};
  vf.B = bsr->B;
  vf.d = d;
  vf.H_kv = H_kv;
  vf.n_brow = bsr->n_brow;
  vf.T = bsr->T;
  vf.frag = reinterpret_cast<uint16_t*>(p);
  vf.exps = reinterpret_cast<int32_t*>(p + kNoAllocFragBytes);
  mf::VprepArgs va{};
  va.V = V;
  va.dtype = dtype_code(vdtype);
  va.H_kv = H_kv;
  va.d = d;
  va.B = bsr->B;
  va.T = bsr->T;
  va.n_brow = bsr->n_brow;
  va.info = bsr->brow_info;            // the store's geometry tables, already on the device
  va.brow_seq = bo->brow_seq;
  va.page_table = page_table;
  va.page_size = page_size;
  va.pages_per_seq = pages_per_seq;
  va.vmax_bits = reinterpret_cast<uint32_t*>(p + kNoAllocFragBytes + 1024);   // cleared by a kernel first
  va.frag = vf.frag;
  va.exps = vf.exps;
  MF_HIP(mf::v_prepare(va, s), "V preparation launch");
  const mf_vfrag* vfp = &vf;
  return retrieve_launch(ctx, bsr, 1, &W, &H_r, &vfp, &kvmap, &O, stream, 0, nullptr, true);
}

MF_EXPORT mf_status mf_copy_probe(mf_ctx* ctx, void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return fail(MF_ERR_INVALID, "dst or src is NULL");
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return fail(MF_ERR_INVALID, "copy probe needs 16-byte aligned pointers and a multiple of 16 bytes");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(mf::copy_probe(dst, src, bytes, static_cast<hipStream_t>(stream)), "copy probe launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_read_probe(mf_ctx* ctx, const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(MF_ERR_INVALID, "src or sink is NULL");
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(MF_ERR_INVALID, "read probe needs a 16-byte aligned source, a multiple of 16 bytes and a 4-byte aligned sink");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(mf::read_probe(src, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)), "read probe launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_write_probe(mf_ctx* ctx, void* dst, size_t bytes, const void* src, void* stream) {
  if (!dst) return fail(MF_ERR_INVALID, "dst is NULL");
  if (bytes % 20480 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return fail(MF_ERR_INVALID, "write probe needs 16-byte aligned pointers and a multiple of 20480 bytes");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(mf::write_probe(dst, bytes, src, static_cast<hipStream_t>(stream)), "write probe launch");
  return MF_OK;
}

MF_EXPORT mf_status mf_fill_probe(mf_ctx* ctx, void* dst, size_t bytes, uint32_t value, void* stream) {
  if (!dst) return fail(MF_ERR_INVALID, "dst is NULL");
  if (bytes % 262144 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15))
    return fail(MF_ERR_INVALID, "fill probe needs a 16-byte aligned destination and a multiple of 262144 bytes");
  mf_status st = set_device(ctx);
  if (st != MF_OK) return st;
  MF_HIP(mf::fill_probe(dst, bytes, value, static_cast<hipStream_t>(stream)), "fill probe launch");
  return MF_OK;
}

}  // extern "C"
