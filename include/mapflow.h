/*
 * mapflow.h — C ABI of libmapflow, the MI355X (gfx950) hot path of MapFlow's cross-model
 * attention-map reuse: block-sparse compression of a sender layer's causal softmax map, and the
 * fused retrieval that turns the kept blocks into a receiver layer's attention output.
 *
 * Page keys cited below:
 *   [MapFlow开源]  "MapFlow开源:大模型换班,Prefill为何能快20%?" (aitest123.com)
 *   [Reuses Attention] "Peking University's MapFlow Reuses Attention Across Models without
 *                   Recomputing the KV Cache" (roboind.com)
 *   [Abstract]     "Accelerating Cross-Model LLM Inference via Attention Map Reuse", abstract
 *
 * Conventions for every call:
 *   - Pointers named *_host are host memory; every other data pointer is device memory on the
 *     context's device.  The library never frees caller memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on it; calls
 *     return before the GPU finishes unless stated otherwise.
 *   - Arguments are validated on the host before anything is launched; a failed check returns
 *     MF_ERR_INVALID (or MF_ERR_UNSUPPORTED for valid shapes the library has no kernel for) and
 *     leaves all outputs untouched.  No C++ exception crosses this boundary.
 *   - After a non-OK status, mf_last_error() returns a message for the calling thread.
 *   - A context holds scratch memory: calls on one context that use the same scratch (two
 *     compresses, or two retrieves through mf_retrieve) must be ordered on one stream.  When a
 *     call needs more scratch than it holds, it waits for its own stream (only that stream) before
 *     handing the old buffer back, then takes a larger one.
 *   - Device memory comes from the allocator given to mf_create (for example PyTorch's caching
 *     allocator), or from hipMalloc / hipFree when none is given.  Every library-owned device
 *     buffer (stores, prepared V, context scratch, cache entries) is taken and returned through it.
 */
#ifndef MAPFLOW_H
#define MAPFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mf_status {
  MF_OK = 0,
  MF_ERR_INVALID = 1,     /* bad argument; nothing launched, outputs untouched */
  MF_ERR_UNSUPPORTED = 2, /* valid request with no compiled kernel (see each call's limits) */
  MF_ERR_OOM = 3,         /* a device allocation failed; nothing leaked */
  MF_ERR_HIP = 4,         /* a HIP runtime call or a kernel launch failed */
  MF_ERR_CAPACITY = 5     /* a preallocated block store was too small for the kept blocks */
} mf_status;

typedef enum mf_dtype { MF_F32 = 0, MF_BF16 = 1 } mf_dtype;

typedef struct mf_ctx mf_ctx;
typedef struct mf_cache mf_cache;

/*
 * Block-sparse (BSR) store of one sender layer's compressed attention map.
 * [MapFlow开源, section 只存重要的:块稀疏压缩]: the map is cut into regular B x B blocks and only
 * the high-mass blocks are stored; the number kept varies per layer and per position.
 *
 * Block rows are numbered over the packed batch: sequence s owns block rows
 * [brow_base(s), brow_base(s) + ceil(n_s / B)); block columns are local to the sequence
 * (column 0 is the sequence's first B tokens).  All arrays are device memory owned by the
 * library (free with mf_bsr_free).
 *
 *   brow_info   int32 [n_brow][4]   {first token of the block row, first token of its sequence,
 *                                     sequence length, block row index within the sequence}
 *   brow_order  int32 [n_order]      the retrieve's work order over the active block rows:
 *                                    descending in-sequence index, dealt in runs of 64 entries
 *                                    so that entry p (run on XCD p mod 8) and its neighbours on
 *                                    that XCD are 8 consecutive rows of the order
 *   brow_coff   int32 [n_brow]       causal blocks of all earlier block rows (exclusive prefix
 *                                    of I + 1): the row's offset in per-causal-block scratch
 *   block_ptr   int32 [n_brow + 1]   CSR row pointer over kept blocks
 *   block_idx   int32 [capacity]     kept block columns, ascending within each block row
 *   block_row   int32 [capacity]     block row of each kept block
 *   probs       bf16  [capacity][ceil(H_s/8)][B][B][8]  kept probabilities; element
 *               [n][h/8][r][c][h%8] is the softmax probability of query row r and key column c
 *               of block n for sender head h, rounded to bf16 (nearest even).  Zero for r or c
 *               past the sequence end, above the causal diagonal, and for padding heads >= H_s.
 *   row_kept_mass fp32 [H_s][T]      per head and token, the sum of that row's stored probs
 *   counters    int32 [2]            {nnzb, overflow flag} written by the device
 */
typedef struct mf_bsr {
  int32_t B;          /* block size (16, 32, 64 or 128)                        */
  int32_t H_s;        /* sender heads                                          */
  int32_t n_seq;      /* sequences in the packed batch                        */
  int32_t n_brow;     /* block rows over all sequences                        */
  int32_t nb_max;     /* largest per-sequence block count                     */
  int32_t n_order;    /* block rows compressed and retrieved (n_brow unless the store was
                         created with a row range by mf_bsr_create_range)              */
  int64_t T;          /* tokens in the packed batch                           */
  int64_t n_causal;   /* causal (lower-triangular) blocks over all sequences  */
  int64_t capacity;   /* blocks allocated in block_idx / block_row / probs    */
  int64_t nnzb;       /* kept blocks; valid after mf_compress or mf_bsr_sync  */
  int32_t* brow_info;
  int32_t* brow_order;
  int32_t* brow_coff;
  int32_t* block_ptr;
  int32_t* block_idx;
  int32_t* block_row;
  uint16_t* probs;
  float* row_kept_mass;
  int32_t* counters;
  void* _owner;       /* library bookkeeping; do not touch                    */
} mf_bsr;

/*
 * Receiver V prepared for the MFMA kernels: fp16, scaled per KV head by 2^exps[k] so the largest
 * |V| of each head sits near 2^15, and laid out so that each 32-key x 16-column operand tile is one
 * contiguous 1 KiB read.  Keys are grouped by B-token block rows exactly as an mf_bsr with the
 * same cu_seqlens and B; rows past a sequence end are zero.
 */
typedef struct mf_vfrag {
  int32_t B, d, H_kv, n_brow;
  int64_t T;
  uint16_t* frag;     /* fp16 [H_kv][n_brow][B/32][d/16][64 lanes][8]            */
  int32_t* exps;      /* int32 [H_kv] power-of-two scale exponents                */
  void* _owner;
} mf_vfrag;

/* Library version string (static storage). */
const char* mf_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* mf_last_error(void);

/*
 * The caller's device allocator.  alloc returns `bytes` (> 0) of device memory on the context's
 * device, aligned to at least 256 bytes, for work enqueued on `stream` (a hipStream_t; NULL = the
 * default stream), or NULL when it cannot; the library then returns MF_ERR_OOM and hands back
 * everything the failing call had taken.  release returns one pointer alloc gave, with the same
 * `bytes`; the library calls it only when no work it enqueued still uses the memory (it has
 * waited for the stream that used it, or for the device).  `user` is passed through unchanged.
 * Both callbacks run on the thread that called into the library.
 */
typedef void* (*mf_alloc_fn)(size_t bytes, void* stream, void* user);
typedef void (*mf_free_fn)(void* ptr, size_t bytes, void* stream, void* user);

/*
 * Create a context on HIP device `device`.  alloc and release are the caller's allocator (both or
 * neither: NULL, NULL means hipMalloc / hipFree); `user` goes to both.  The context keeps scratch
 * memory taken from that allocator.  Stores and prepared V created on the context keep a copy of
 * the allocator, so they may be freed after the context is destroyed (with ctx = NULL).
 */
mf_status mf_create(int device, mf_alloc_fn alloc, mf_free_fn release, void* user, mf_ctx** out);

/* Destroy a context and return its scratch memory (after synchronising the device). */
mf_status mf_destroy(mf_ctx* ctx);

/*
 * Install the layer map that mf_prefill_layers follows (host only: validates and copies).
 * [MapFlow开源, section 不传 KV Cache,改传'注意力关系']: a sender layer's map is assigned to a
 * suitable receiver layer; [Reuses Attention] and [Abstract]: the receiver computes its first
 * layers itself (partial recomputation).  pi_host int32 [n_recv]: pi[l] = -1 exactly for l < R
 * (receiver layer l is recomputed with dense causal attention), otherwise the sender layer in
 * [0, n_send) whose compressed map receiver layer l reuses.  MF_ERR_INVALID otherwise (the
 * context's previous map is kept).
 */
mf_status mf_map_layers(mf_ctx* ctx, const int32_t* pi_host, int32_t n_recv, int32_t n_send, int32_t R);

/*
 * A uniform layer map (host only, needs no GPU): pi_out[l] = -1 for l < R, otherwise
 * round(l * (n_send - 1) / (n_recv - 1)) with halves rounded up, computed in integers (0 when
 * n_recv = 1).  Requires n_recv >= 1, n_send >= 1, 0 <= R <= n_recv.
 */
mf_status mf_layer_map_uniform(int32_t n_recv, int32_t n_send, int32_t R, int32_t* pi_out_host);

/*
 * Check a layer map without installing it: pi[l] == -1 exactly for l < R and 0 <= pi[l] < n_send
 * otherwise.  Host only.
 */
mf_status mf_check_layer_map(const int32_t* pi_host, int32_t n_recv, int32_t n_send, int32_t R);

/*
 * Allocate an empty block store for a packed batch: geometry from cu_seqlens_host (int32
 * [n_seq + 1], non-decreasing, starting at 0) and block size B.  capacity_blocks < 0 allocates
 * room for every causal block, so any tau fits.  H_s in [1, 64].
 */
mf_status mf_bsr_create(mf_ctx* ctx, int32_t H_s, int32_t B, const int32_t* cu_seqlens_host,
                        int32_t n_seq, int64_t capacity_blocks, mf_bsr* out);

/*
 * A block store for chunked prefill: like mf_bsr_create, but only block rows I >= row_begin[s]
 * of each sequence s are compressed and retrieved (row_begin_host: int32 [n_seq], each in
 * [0, ceil(n_s / B)]).  [MapFlow开源, section 算得省的:融合内核执行] names chunked prefill among
 * the serving features the retrieval works with; rows of an earlier chunk come from another
 * store, for example a cached prefix (mf_cache_lookup).  Every row still exists as a key block
 * row, so Q and K (and V for the retrieve) are passed for the whole sequence as usual; row
 * selection, probabilities and kept mass of a compressed row are exactly those of the same row
 * in an mf_bsr_create store.  Rows outside the range keep no blocks, their kept mass is 0, and
 * mf_retrieve* / mf_compress_prefill_into leave their output rows untouched.
 * capacity_blocks < 0 allocates every causal block of the compressed rows.
 */
mf_status mf_bsr_create_range(mf_ctx* ctx, int32_t H_s, int32_t B, const int32_t* cu_seqlens_host,
                              int32_t n_seq, const int32_t* row_begin_host, int64_t capacity_blocks,
                              mf_bsr* out);

/*
 * Copy a store to host memory (synchronous; waits for the device).  Any destination may be NULL
 * to skip it.  block_ptr_host: int32 [n_brow + 1]; block_idx_host: int32 [nnzb]; probs_host:
 * bf16 bits in the store layout, [nnzb][ceil(H_s/8)][B][B][8]; row_kept_mass_host: fp32 [H_s][T].
 * nnzb is read from the device first (bsr->nnzb is updated).
 */
mf_status mf_bsr_download(mf_ctx* ctx, mf_bsr* bsr, int32_t* block_ptr_host,
                          int32_t* block_idx_host, uint16_t* probs_host,
                          float* row_kept_mass_host);

/*
 * Copy the kept blocks [first, first + count) of a store to host memory (synchronous; waits for
 * the device): block_idx_host int32 [count] and probs_host bf16 bits [count][ceil(H_s/8)][B][B][8]
 * (either may be NULL).  The range must lie inside [0, nnzb) of the device's kept-block count;
 * MF_ERR_INVALID otherwise.  Lets a caller inspect part of a store that does not fit the host.
 */
mf_status mf_bsr_download_blocks(mf_ctx* ctx, mf_bsr* bsr, int64_t first, int64_t count,
                                 int32_t* block_idx_host, uint16_t* probs_host);

/*
 * Fill a store from host memory (synchronous), e.g. to restore a store saved with
 * mf_bsr_download from a host-memory tier.  Same layouts as mf_bsr_download.  block_ptr_host
 * must start at 0, be non-decreasing and end at nnzb <= capacity; each block row's columns must
 * be ascending and within [0, I] of that row.  Checked on the host; MF_ERR_INVALID otherwise.
 */
mf_status mf_bsr_upload(mf_ctx* ctx, mf_bsr* bsr, const int32_t* block_ptr_host,
                        const int32_t* block_idx_host, const uint16_t* probs_host,
                        const float* row_kept_mass_host);

/*
 * Free the device arrays of a store created by this library and zero *bsr.  The device is
 * synchronised first (no enqueued work may still read or write the arrays), then the memory goes
 * back through the allocator the store was created with.  ctx may be NULL (for example after
 * mf_destroy); a store that a prefix cache owns is refused with MF_ERR_INVALID.
 */
mf_status mf_bsr_free(mf_ctx* ctx, mf_bsr* bsr);

/*
 * Compress one sender layer into an existing store (no allocation on the store, no host sync).
 * [MapFlow开源, section 只存重要的:块稀疏压缩] and [Reuses Attention, first component]: block
 * statistics first, then the kept blocks; the dense L x L map is never formed.
 *
 *   Q, K   sender queries and keys, [H_s][T][d] (head-major, post-RoPE), dtype MF_BF16 or MF_F32;
 *          device pointers, 16-byte aligned (MF_ERR_INVALID otherwise)
 *   d      64 or 128
 *   tau    in (0, 1]: per block row, keep the sink block (column 0) and the diagonal block, then
 *          blocks by descending mass (ties: lower column) until the kept mass reaches
 *          tau * H_s * rows; tau = 1 keeps every causal block
 * Scores are q.k / sqrt(d).  If the kept blocks exceed bsr->capacity, the store's overflow flag
 * is set and the extra blocks are dropped; mf_bsr_sync reports it as MF_ERR_CAPACITY.
 * Scratch memory of the context may grow (a device allocation) on the first call of a size.
 */
mf_status mf_compress_into(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype, int32_t d,
                           float tau, mf_bsr* bsr, void* stream);

/*
 * The sender's own prefill attention and the compression of its map in one pass over the scores.
 * [MapFlow开源, section 只存重要的:块稀疏压缩]: the map is compressed without first assembling the
 * dense matrix; here the score tiles that the sender's causal attention forms anyway also give
 * the block statistics, so no separate statistics pass runs.
 * Fills *bsr as mf_compress_into(ctx, Q, K, dtype, d, tau, bsr, stream) does, up to rounding
 * (mf_compress_into sums most blocks' statistics against the row's running maximum, this call
 * against each block's own maximum; block choices can differ only at near-ties of the masses),
 * and also writes
 *     O[i, h, :] = sum_j softmax_j(q_i . k_j / sqrt(d), j <= i within i's sequence) V[j, h, :]
 *   Q, K   [H_s][T][d] as for mf_compress_into
 *   V      sender values, [T][H_s][d] (one value head per sender head), dtype as Q; 16-byte aligned
 *   O      fp32 [T][H_s][d] device; must not alias any input
 * Probabilities enter the P.V product as fp16 scaled by 2^15 and V as fp16 with a power-of-two
 * scale per head (as in mf_dense_attention); sums are fp32.  The prepared V lives in context
 * scratch (may allocate on the first call of a size).  Errors as mf_compress_into, plus
 * MF_ERR_INVALID for a NULL V or O.
 */
mf_status mf_compress_prefill_into(mf_ctx* ctx, const void* Q, const void* K, const void* V,
                                   mf_dtype dtype, int32_t d, float tau, mf_bsr* bsr, float* O,
                                   void* stream);

/*
 * Variants of the compression that the pages' wording allows ([MapFlow 方案, 二]: cross-layer and
 * cross-head linear mapping; [MapFlow开源, the head-mapping bullet]).  Option bits:
 *   MF_SELECT_PER_HEAD  every sender head selects its own blocks (forced sink and diagonal, then
 *                       its own block masses in descending order until tau * rows); the store
 *                       keeps the union, and a head stores zeros in blocks it did not select
 *   MF_NORM_PER_HEAD    each head's kept row is divided by that head's mass over its kept blocks
 *                       before rounding to bf16 (so each head's stored row sums to ~1); the
 *                       retrieve then mixes the normalised heads and renormalises as usual
 * options = 0 is mf_compress_into.  The store layout and every retrieve call are unchanged.
 */
enum { MF_SELECT_PER_HEAD = 1, MF_NORM_PER_HEAD = 2 };
mf_status mf_compress_into_ex(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype, int32_t d,
                              float tau, uint32_t options, mf_bsr* bsr, void* stream);

/* Wait for `stream`, read the kept-block count into bsr->nnzb; MF_ERR_CAPACITY on overflow. */
mf_status mf_bsr_sync(mf_ctx* ctx, mf_bsr* bsr, void* stream);

/*
 * Compress with an exactly sized store: the selection runs first, the stream is synchronised
 * once to read the kept-block count, then block_idx / probs are allocated for exactly nnzb
 * blocks and filled.  *out must be freed with mf_bsr_free.  Same arguments as mf_compress_into
 * plus the geometry of mf_bsr_create.
 */
mf_status mf_compress(mf_ctx* ctx, const void* Q, const void* K, mf_dtype dtype, int32_t H_s,
                      int32_t d, const int32_t* cu_seqlens_host, int32_t n_seq, float tau,
                      int32_t B, void* stream, mf_bsr* out);

/*
 * Prepare the receiver's V for retrieval (and for mf_dense_attention).
 *   V            contiguous [T][H_kv][d] when page_table is NULL; otherwise a page pool
 *                [n_pages][page_size][H_kv][d] with page_table int32 [n_seq][pages_per_seq]
 *                (device) mapping each sequence's logical pages to pool pages; V is a device
 *                pointer, 16-byte aligned (MF_ERR_INVALID otherwise)
 *   dtype        MF_BF16 or MF_F32
 * If out->frag is NULL the library allocates frag and exps (free with mf_vfrag_free); otherwise
 * the caller provides frag with room for H_kv * n_brow * B * d fp16 values.  Calling again with an
 * already prepared *out of the same geometry re-prepares in place without allocating.
 * Values scaled past the fp16 range are not possible: each head is scaled by 2^e with
 * max|V| * 2^e <= 2^15.  Non-finite V propagates as in IEEE arithmetic.
 */
mf_status mf_v_prepare(mf_ctx* ctx, const int32_t* cu_seqlens_host, int32_t n_seq, int32_t B,
                       const void* V, mf_dtype dtype, int32_t H_kv, int32_t d,
                       const int32_t* page_table, int32_t page_size, int32_t pages_per_seq,
                       mf_vfrag* out, void* stream);

/*
 * Free what the library allocated for prepared V (its geometry tables and exponents, and frag
 * unless the caller provided it) and zero *vf; caller-provided frag memory is left alone.  Same
 * rules as mf_bsr_free: the device is synchronised first, the memory goes back through the
 * allocator it came from, ctx may be NULL.
 */
mf_status mf_vfrag_free(mf_ctx* ctx, mf_vfrag* vf);

/*
 * Fused retrieve on a prepared V.  [MapFlow开源, section 算得省的:融合内核执行] and
 * [Reuses Attention, third component]: read the kept blocks, combine sender heads into receiver
 * heads on chip, multiply by the receiver's own V, accumulate, write the output — no dense map
 * and no mixed map in device memory.  For receiver head g and token i:
 *     Ahat[g,i,j] = sum_h W[g,h] P[h,i,j] over kept keys j,
 *     O[i,g,:]    = sum_j Ahat[g,i,j] V[j, kv(g), :] / sum_j Ahat[g,i,j].
 *   W                 fp32 [H_r][H_s] device, any real values (not validated; a zero row sum
 *                     gives IEEE inf/nan like the definition)
 *   kv_head_map_host  int32 [H_r], each in [0, H_kv)
 *   O                 fp32 [T][H_r][d] device; must not alias any input
 * Limits: H_r <= 48, H_s <= 64, d in {64, 128}, B in {32, 64}, vf geometry equal to the store's.
 * Above 24 receiver heads the heads are mixed by two workgroups per row tile (equal halves),
 * each reading the tile (the second read is served by L2), except for a receiver of exactly 32
 * heads at B = 64 whose KV heads each serve a multiple of 4 query heads: one workgroup mixes all
 * 32, taking each kept block as two 32-key halves.
 * Rows of the mixed map are rounded to fp16 (scaled by a power of two per receiver head) before
 * the V product; sums are fp32.
 */
mf_status mf_retrieve_prepared(mf_ctx* ctx, const mf_bsr* bsr, const float* W, int32_t H_r,
                               const mf_vfrag* vf, const int32_t* kv_head_map_host, float* O,
                               void* stream);

/*
 * Fused retrieve for several receivers of one sender state in a single launch.
 * [MapFlow开源, section 多模型工作流端到端加速] and [Reuses Attention, the three-model workflow
 * paragraph]: two downstream models share the attention state one upstream model produced.
 * Receiver r computes exactly what mf_retrieve_prepared(ctx, bsr, W[r], H_r[r], vf[r],
 * kv_head_map_host[r], O[r], stream) computes, bit for bit; the launch reads each kept block of
 * the store from device memory once for all receivers instead of once per receiver.
 *   n_recv            1..4
 *   W, H_r, vf, kv_head_map_host, O   host arrays of n_recv entries; entry r has the meaning,
 *                     layout and limits of the same argument of mf_retrieve_prepared
 * All receivers share the head dimension d.  Each receiver's heads, in KV-head order, form one
 * part of at most 24 heads, or two equal parts above 24 (a 32-head receiver that one workgroup
 * mixes alone, as described for mf_retrieve_prepared, stays one part with a workgroup of its
 * own); parts are packed first-fit, largest first, into workgroups of at most 24 heads per row
 * tile (a workgroup may hold parts of several receivers), with one launch per width (heads per
 * wave).  Outputs must not alias each other or
 * any input.  Validation happens before any launch: on an error nothing is written.
 */
mf_status mf_retrieve_multi(mf_ctx* ctx, const mf_bsr* bsr, int32_t n_recv, const float* const* W,
                            const int32_t* H_r, const mf_vfrag* const* vf,
                            const int32_t* const* kv_head_map_host, float* const* O,
                            void* stream);

/*
 * One receiver layer from the stores of several sender layers (a variant the wording allows:
 * [MapFlow 方案, 二] names a linear mapping across layers as well as heads).  For receiver head
 * g and token i, with P_l zero outside layer l's kept blocks:
 *     Ahat[g,i,j] = sum_l sum_h W_l[g,h] P_l[h,i,j],   O[i,g,:] = sum_j Ahat V / sum_j Ahat,
 * i.e. mf_retrieve_prepared over the union of the layers' blocks.  stores: n_layers stores with
 * the same B, cu_seqlens and row range (H_s may differ); W[l]: fp32 [H_r][stores[l].H_s] device;
 * vf, kv_head_map_host, O as for mf_retrieve_prepared.  One launch per layer; O holds the running
 * unnormalised sum in between and the context keeps the running denominators [T][H_r].
 * n_layers = 1 is mf_retrieve_prepared.
 */
mf_status mf_retrieve_layers(mf_ctx* ctx, int32_t n_layers, const mf_bsr* stores, const float* const* W,
                             int32_t H_r, const mf_vfrag* vf, const int32_t* kv_head_map_host, float* O,
                             void* stream);

/* mf_v_prepare into context scratch followed by mf_retrieve_prepared. */
mf_status mf_retrieve(mf_ctx* ctx, const mf_bsr* bsr, const float* W, int32_t H_r, const void* V,
                      mf_dtype vdtype, int32_t H_kv, int32_t d, const int32_t* page_table,
                      int32_t page_size, int32_t pages_per_seq, const int32_t* kv_head_map_host,
                      float* O, void* stream);

/*
 * mf_retrieve without any device allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, result and error codes as mf_retrieve, bit for bit.  The prepared V goes into
 * a fixed device array of the library (64 MiB + 4 KiB per device, held until the process ends)
 * instead of context scratch, and the geometry tables come from the store itself; no hipMalloc,
 * hipFree or allocator callback is called.  Limit: H_kv * n_brow * B * d <= 2^25 fp16 values
 * (e.g. 32768 tokens of one sequence with 8 KV heads at d = 128), else MF_ERR_UNSUPPORTED before
 * anything is launched.  Every call on a device shares that device's array and overwrites what
 * the previous call left there (the per-head maxima are cleared by a kernel at the start of each
 * call): two calls that overlap on one device, on any streams or contexts, race and give wrong
 * outputs.  Order them on one stream.
 */
mf_status mf_retrieve_noalloc(mf_ctx* ctx, const mf_bsr* bsr, const float* W, int32_t H_r, const void* V,
                              mf_dtype vdtype, int32_t H_kv, int32_t d, const int32_t* page_table,
                              int32_t page_size, int32_t pages_per_seq, const int32_t* kv_head_map_host,
                              float* O, void* stream);

/*
 * Dense causal attention for the receiver layers that are recomputed ([Reuses Attention]:
 * the receiver computes its first layers normally).  O[i,g,:] = softmax_j<=i(q.k / sqrt(d)) V
 * per sequence, query head g reading KV head kv_head_map_host[g].
 *   Q [T][H_q][d], K, V [T][H_kv][d] (MF_BF16 or MF_F32), O fp32 [T][H_q][d]; d in {64, 128}.
 *   Q, K and V must be 16-byte aligned (MF_ERR_INVALID otherwise).
 */
mf_status mf_dense_attention(mf_ctx* ctx, const void* Q, const void* K, const void* V,
                             mf_dtype dtype, int32_t H_q, int32_t H_kv, int32_t d,
                             const int32_t* cu_seqlens_host, int32_t n_seq,
                             const int32_t* kv_head_map_host, float* O, void* stream);

/*
 * One receiver prefill over every layer: partial recomputation plus map reuse, with the prefetch
 * of later layers' blocks overlapped with the recomputation of the first layers.
 * [Reuses Attention]: the receiver computes its first few layers itself; [MapFlow开源, section
 * 2. 找得快的:基于前缀哈希的缓存管理]: while those layers compute, the attention blocks that later
 * layers need are already being loaded asynchronously in the background; [MapFlow开源, section
 * 3. 算得省的:融合内核执行]: each reused layer runs the fused retrieve.
 *
 * The layer map is the one installed by mf_map_layers (n_recv receiver layers, n_send sender
 * layers, the first R recomputed).  The m-th mapped receiver layer l (in layer order) reuses sender
 * layer pi[l], compressed into ring slot m % n_slots.  Two streams:
 *   stream_prefetch  compresses the sender layers of the first n_slots mapped layers, then each
 *                    later one as soon as the retrieve that last read its slot has finished;
 *   stream_main      runs dense causal attention for layers 0..R-1 (beside the first
 *                    compresses), then for each mapped layer waits for its slot's compress,
 *                    prepares its V (context scratch) and runs the fused retrieve into its O.
 * HIP events order the two streams; nothing waits on the host.  Both streams start after the work
 * enqueued on stream_main before the call, and stream_main's later work runs after every launch
 * of the call (stream_main waits for stream_prefetch's last compress at the end).
 * flags:
 *   MF_PREFILL_ISOLATE  each retrieve also waits until stream_prefetch is idle, and each later
 *                       compress waits for that retrieve, so a retrieve never shares the GPU with
 *                       a compress (the retrieve's event time is then its kernel time)
 *   MF_PREFILL_TIMING   record timing events; read them with mf_prefill_timings
 *
 *   recv            host array of n_recv entries, in receiver layer order:
 *                     layers l < R: Q [T][H_r][d], K and V [T][H_kv][d], O fp32 [T][H_r][d];
 *                     mapped layers: V [T][H_kv][d], W fp32 [H_r][H_s], O fp32 [T][H_r][d]
 *                     (Q and K unused)
 *   send            host array of n_send entries: sender queries and keys [H_s][T][d]; only the
 *                   entries some pi[l] names are read
 *   dtype           MF_BF16 or MF_F32, for every Q, K and V
 *   kv_head_map_host int32 [H_r]: KV head of each receiver query head (all layers)
 *   tau             in (0, 1], as for mf_compress_into
 *   slots           n_slots >= 1 stores from mf_bsr_create with one geometry (cu_seqlens, B, H_s),
 *                   not range stores or cache views, each with capacity for every causal block
 *                   (capacity_blocks < 0), so no compress in the ring can overflow
 * Every Q, K and V must be 16-byte aligned.  The limits of mf_compress_into, mf_retrieve_prepared
 * and mf_dense_attention apply.  All arguments are validated before anything is launched.  After
 * the call the slots hold the last n_slots mapped layers' stores.  Two calls on one context must
 * not overlap (they share the prepared-V scratch and the events).
 */
typedef struct mf_recv_layer {
  const void* Q;
  const void* K;
  const void* V;
  const float* W;
  float* O;
} mf_recv_layer;

typedef struct mf_send_layer {
  const void* Q;
  const void* K;
} mf_send_layer;

enum { MF_PREFILL_ISOLATE = 1, MF_PREFILL_TIMING = 2 };
mf_status mf_prefill_layers(mf_ctx* ctx, const mf_recv_layer* recv, const mf_send_layer* send,
                            mf_dtype dtype, int32_t H_r, int32_t H_kv, int32_t d,
                            const int32_t* kv_head_map_host, float tau, int32_t n_slots,
                            mf_bsr* slots, uint32_t flags, void* stream_main,
                            void* stream_prefetch);

/*
 * Stage times of the last mf_prefill_layers call made with MF_PREFILL_TIMING, in milliseconds
 * (waits for that call to finish).  Each output may be NULL:
 *   dense_ms     [R]      dense attention of receiver layers 0..R-1
 *   compress_ms  [n_map]  compress of the m-th mapped layer's sender layer (stream_prefetch)
 *   vprep_ms     [n_map]  V preparation of the m-th mapped layer (stream_main)
 *   retrieve_ms  [n_map]  fused retrieve of the m-th mapped layer (stream_main)
 * n_map = n_recv - R of the installed layer map.  MF_ERR_INVALID if no timed call was made.
 */
mf_status mf_prefill_timings(mf_ctx* ctx, float* dense_ms_host, float* compress_ms_host,
                             float* vprep_ms_host, float* retrieve_ms_host);

/*
 * Prefix-hash cache of compressed sender state.  [MapFlow开源, section 找得快的:基于前缀哈希的缓存管理]
 * and [Reuses Attention, second component]: the sparse blocks kept per layer and position vary in
 * number; they are indexed by a hash that carries the preceding context, so a receiver reusing
 * the state finds its blocks through that index.
 *
 * mf_prefix_hashes (host only): for each full block r of B tokens (r < n_tokens / B),
 *     h_{-1} = FNV1a64(4 little-endian bytes of B),
 *     h_r    = FNV1a64(8 little-endian bytes of h_{r-1} || 4 little-endian bytes of each token of
 *              block r),
 * FNV-1a 64-bit with offset basis 0xcbf29ce484222325 and prime 0x100000001b3, restarted from the
 * offset basis for every h_r.  h_r depends on every token up to the end of block r and on B, so it
 * names a block row's compressed content, which depends on exactly those tokens.
 */
mf_status mf_prefix_hashes(const int32_t* tokens_host, int64_t n_tokens, int32_t B, uint64_t* hashes_out);

/*
 * A cache of compressed token prefixes in device memory, at most budget_bytes (entries are
 * evicted least recently used first).  Not thread-safe: one thread uses a cache at a time.
 */
mf_status mf_cache_create(mf_ctx* ctx, int64_t budget_bytes, mf_cache** out);
/* Synchronises the device, frees every entry (views from mf_cache_lookup become invalid). */
mf_status mf_cache_destroy(mf_cache* cache);
/* Number of entries and bytes held. */
mf_status mf_cache_info(const mf_cache* cache, int64_t* entries, int64_t* used_bytes);

/*
 * Cache block rows 0..rows-1 of one sequence for `layer`, keyed by (layer, rows, h_{rows-1}) of
 * tokens_host[0 .. n_tokens) and confirmed by the tokens themselves on lookup.  Each row is copied
 * (device to device, on `stream`, which is synchronised) from the first of parts[0 .. n_parts)
 * that compressed it completely: parts are single-sequence stores of the same B and H_s whose
 * token 0 is token 0 of tokens_host (a store of the whole sequence, or a looked-up prefix and a
 * mf_bsr_create_range store of the rows after it).  MF_ERR_INVALID when a row is in no part;
 * MF_ERR_CAPACITY when the entry alone exceeds the budget.  Inserting an existing prefix only
 * refreshes it.  May evict other entries, invalidating their views.
 */
mf_status mf_cache_insert(mf_cache* cache, int32_t layer, const int32_t* tokens_host, int64_t n_tokens,
                          int32_t n_parts, const mf_bsr* parts, int32_t rows, void* stream);

/*
 * Longest cached prefix of tokens_host for `layer` with block size B: *rows_out = its block rows
 * (0 when nothing matches) and *view_out = a store of exactly those rows (one sequence of
 * rows * B tokens), owned by the cache: read it (mf_retrieve*, mf_bsr_download, as a part of
 * mf_cache_insert), never free it (mf_bsr_free refuses); valid until evicted or the cache is
 * destroyed.  The rows after it are compressed with an mf_bsr_create_range store.
 */
mf_status mf_cache_lookup(mf_cache* cache, int32_t layer, const int32_t* tokens_host, int64_t n_tokens,
                          int32_t B, int32_t* rows_out, mf_bsr* view_out);

/*
 * HBM probe: copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to dst with
 * a plain streaming kernel.  Used to calibrate bandwidth counters against a known byte count.
 */
mf_status mf_copy_probe(mf_ctx* ctx, void* dst, const void* src, size_t bytes, void* stream);

/*
 * HBM read probe: read `bytes` (a multiple of 16, src 16-byte aligned) with non-temporal 16-byte
 * loads and fold them by XOR; `sink` (4 bytes of device memory, 4-byte aligned) is written only
 * if a thread's fold equals one fixed 128-bit value (so the loads cannot be optimised away), and
 * nothing else is written.  Gives the read ceiling that a read-dominated kernel such as the
 * fused retrieve is compared with.
 */
mf_status mf_read_probe(mf_ctx* ctx, const void* src, size_t bytes, void* sink, void* stream);

/*
 * HBM write probe: write `bytes` (a multiple of 20480; dst 16-byte aligned) to dst with coalesced
 * non-temporal 16-byte stores, 1 KiB of contiguous memory per wavefront instruction.  With src
 * (16-byte aligned, bytes / 5 readable) it first reads bytes / 5 from src with non-temporal
 * loads, one 16-byte record per five written: the read : write mix of the block gather of
 * mf_compress, whose writes of kept probabilities outweigh its key reads about five to one.
 * Record it * 1280 + 256 u + t of dst (u = 0..4, t = 0..255) receives src record it * 256 + t, or
 * {it, 7, 8, 9} without src, plus u in each 32-bit word.  src may be NULL.  Gives the write-heavy
 * ceiling that the gather is compared with.
 */
mf_status mf_write_probe(mf_ctx* ctx, void* dst, size_t bytes, const void* src, void* stream);

/*
 * HBM fill probe: write `value` to every 32-bit word of dst (`bytes` a multiple of 262144, dst
 * 16-byte aligned) with plain (temporal) 16-byte stores, each workgroup writing 256 KiB of
 * contiguous memory at a time.  Reads nothing.  Gives the device's write ceiling: the
 * non-temporal stores of mf_write_probe (the gather's store kind, which keeps its key tiles in
 * L2) reach less.
 */
mf_status mf_fill_probe(mf_ctx* ctx, void* dst, size_t bytes, uint32_t value, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAPFLOW_H */
