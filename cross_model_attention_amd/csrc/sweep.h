// The score sweep shared by the block statistics (compression), the fused sender prefill and
// the dense causal attention of recomputed layers.
//
// [MapFlow开源, section 只存重要的:块稀疏压缩] (aitest123.com): block-level statistics of the
// attention map are computed without assembling it.  The same sweep, with V, is plain causal
// softmax attention ([Reuses Attention, attention-map section]: the receiver recomputes its first
// layers normally).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mf {

// One lane's slice of a 16-row x D operand tile (rows are queries or keys, K-dim = head dim).
template <typename T, int D>
struct Frag;

template <int D>
struct Frag<uint16_t, D> {
  static constexpr int N = D / 32;
  v8s v[N];
  __device__ __forceinline__ void load(const uint16_t* row, bool valid, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = valid ? as_v8s(ld16(row + 32 * k + 8 * a)) : as_v8s(zero_u4());
  }
};

template <int D>
struct Frag<float, D> {
  static constexpr int N = D / 4;
  float v[N];
  __device__ __forceinline__ void load(const float* row, bool valid, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = valid ? row[4 * k + a] : 0.f;
  }
};

// acc += A B^T over the head dimension, A and B both 16-row fragments.
template <int D>
__device__ __forceinline__ v4f dot_tile(const Frag<uint16_t, D>& A, const Frag<uint16_t, D>& B, v4f acc) {
#pragma unroll
  for (int k = 0; k < Frag<uint16_t, D>::N; ++k) acc = mfma_bf16(A.v[k], B.v[k], acc);
  return acc;
}
template <int D>
__device__ __forceinline__ v4f dot_tile(const Frag<float, D>& A, const Frag<float, D>& B, v4f acc) {
#pragma unroll
  for (int k = 0; k < Frag<float, D>::N; ++k) acc = mfma_f32(A.v[k], B.v[k], acc);
  return acc;
}

constexpr float kNegInf = -__builtin_inff();

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

template <int D>
__device__ __forceinline__ void load_lds_frag(Frag<uint16_t, D>& f, const unsigned char* row, int a) {
#pragma unroll
  for (int k = 0; k < Frag<uint16_t, D>::N; ++k)
    f.v[k] = as_v8s(*reinterpret_cast<const v4u*>(row + (32 * k + 8 * a) * 2));
}
// bf16 key tiles staged by LDS DMA: rows of D bf16 values without padding, 16-byte chunk j of row
// r stored at chunk position j ^ kswz(r); kswz takes 16 distinct values over any 16 consecutive
// rows' bank offsets, so the 16 lanes reading one chunk index of 16 rows hit distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  constexpr int RPB = 256 / (D * 2);                      // rows per 256 bytes (all 64 banks)
  constexpr int NCH = D * 2 / 16;                         // chunks per row
  return (r / RPB) % NCH;
}
template <int D>
__device__ __forceinline__ void load_lds_frag_swz(Frag<uint16_t, D>& f, const unsigned char* tile, int r, int a) {
  const unsigned char* row = tile + r * D * 2;
  const int x = kswz<D>(r);
#pragma unroll
  for (int k = 0; k < Frag<uint16_t, D>::N; ++k)
    f.v[k] = as_v8s(*reinterpret_cast<const v4u*>(row + ((4 * k + a) ^ x) * 16));
}

template <int D>
__device__ __forceinline__ void load_lds_frag(Frag<float, D>& f, const unsigned char* row, int a) {
#pragma unroll
  for (int k = 0; k < Frag<float, D>::N; ++k) f.v[k] = *reinterpret_cast<const float*>(row + (4 * k + a) * 4);
}


// ------------------------------------------------------------------------------------------
// k_stats: one workgroup per (pair of consecutive block rows I, I+1 of one sequence, sender
// head), 2 B/32 waves; the waves of each row own 32 of its queries (two 16-query tiles), so each
// key fragment read from LDS serves 32 queries, and each key tile staged in LDS serves both rows.
// One pass over the key blocks 0..I+1: each block's key tile is staged in LDS (fetched two
// blocks ahead, double buffered), scores are formed transposed (keys x queries) on MFMA, and for
// every (query i, key block J) the block-local maximum r_iJ and z_iJ = sum_{j in J} 2^(s_ij c -
// r_iJ) are stored (c folds log2(e) / sqrt(d)), while each lane keeps the running row logsumexp
// (fp64) of its queries.  Exactly as a softmax over the row would:
//     lse2_i   = log2 sum_J z_iJ 2^(r_iJ)                       (row logsumexp, base 2)
//     M_h[I,J] = sum_{i in I} z_iJ 2^(r_iJ - lse2_i)            (block mass of head h)
// the second sum in fp64, one coalesced read of the stored pairs per block and wave: one
// exponential per score instead of two, and one score pass instead of two.
// ------------------------------------------------------------------------------------------
// Statistics of one (query, key block) pair from the transposed score tiles s[mt] (lane (a, c):
// keys 16 mt + 4 a + i of the block, query c): block maximum r (scaled, base 2) and
// z = sum_j 2^(s_j c - r).  MASKED: keys with (key - query) > 0 are invisible, as is every key of
// a query beyond the sequence; kq = first key of the lane minus the query.
template <int MT, bool MASKED, bool KEEP = false>
__device__ __forceinline__ float2 block_stats(v4f (&s)[MT], int kq, bool qvalid, float scale2) {
  if (MASKED) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!(qvalid && kq + 16 * mt + i <= 0)) s[mt][i] = kNegInf;
  }
  float bm = kNegInf;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    bm = __builtin_fmaxf(bm, __builtin_fmaxf(__builtin_fmaxf(s[mt][0], s[mt][1]), __builtin_fmaxf(s[mt][2], s[mt][3])));
  bm = xrow_max(bm);
  const bool none = MASKED && bm == kNegInf;            // nothing visible: z = 0
  const float r = none ? 0.f : bm * scale2;
  float z = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(fmaf(s[mt][i], scale2, -r));
      z += e;
      if (KEEP) s[mt][i] = e;                           // 2^(s c - r): 0 for invisible keys
    }
  z = xrow_sum(z);
  return make_float2(z, none ? kNegInf : r);
}

// The same for a sweep with the attention half: the reference is the row's new running maximum
// max(m_run, block maximum), so every value stays at most 2^15 in fp16, and s[] receives the
// block's probabilities already scaled for the fp16 products, 2^(s c - ref + 15).  Returns z
// (without the 2^15) and the reference; (0, -inf) when no key of the block is visible.
template <int MT, bool MASKED>
__device__ __forceinline__ float2 block_stats_run(v4f (&s)[MT], int kq, bool qvalid, float scale2, float m_run) {
  if (MASKED) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!(qvalid && kq + 16 * mt + i <= 0)) s[mt][i] = kNegInf;
  }
  float bm = kNegInf;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    bm = __builtin_fmaxf(bm, __builtin_fmaxf(__builtin_fmaxf(s[mt][0], s[mt][1]), __builtin_fmaxf(s[mt][2], s[mt][3])));
  bm = xrow_max(bm);
  const bool none = MASKED && bm == kNegInf;            // nothing visible: z = 0
  const float ref = none ? 0.f : __builtin_fmaxf(m_run, bm * scale2);
  const float off = 15.f - ref;
  float z = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(fmaf(s[mt][i], scale2, off));
      z += e;
      s[mt][i] = e;                                     // 0 for invisible keys
    }
  z = xrow_sum(z);
  return make_float2(z * 0x1p-15f, none ? kNegInf : ref);
}

// Output half of a sweep that also computes attention (the fused sender prefill, and the dense
// recompute): prepared V operand tiles and their per-head exponents.
struct AttnOut {
  const uint16_t* vfrag;
  const int32_t* vexps;
};

// The rows one sweep workgroup reads and writes, by packed token index t: query row q + t q_stride,
// key row k + t k_stride, output row o + t o_stride (fp32, D values); V tiles of head vhead.
template <typename T>
struct SweepHead {
  const T* q;
  int64_t q_stride;
  const T* k;
  int64_t k_stride;
  int vhead;
  float* o;
  int64_t o_stride;
};

// One workgroup of the sweep over the key blocks of a pair of block rows, for one head.  STATS:
// write the block statistics, the row logsumexp and the per-head block masses of head h.  ATTN:
// also accumulate the causal attention output with the same running maximum.
template <typename T, int B, int D, bool ATTN, bool STATS>
__device__ __forceinline__ void sweep_body(const SweepHead<T>& hd, int h, int pr, int64_t T_tot,
                                           const int32_t* __restrict__ info,
                                           const int32_t* __restrict__ pairs,
                                           const int32_t* __restrict__ coff, int64_t n_causal,
                                           int n_brow, int nb_max, float scale2,
                                           float2* __restrict__ zbuf, float* __restrict__ lse2,
                                           float* __restrict__ Mh, AttnOut ao) {
  constexpr int WR = B / 32;                               // waves per block row
  constexpr int MT = B / 16;                               // 16-key tiles per block
  constexpr int QT = 2;                                    // 16-query tiles per wave
  constexpr int NTHR = B * 4;
  // bf16 keys: staged by LDS DMA in the swizzled layout (no registers on the way); fp32 keys:
  // through registers into rows padded to 32 mod 128 bytes
  constexpr bool DMA = sizeof(T) == 2;
  constexpr int ROWB = DMA ? D * 2 : D * (int)sizeof(T) + 32;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int CPT = DMA ? 1 : B * CPR / NTHR;
  constexpr int NDMA = B * D * 2 / 1024 / (NTHR / 64);     // 1 KiB DMA loads per wave and tile
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][B * ROWB];
  __shared__ float s_lse[2][B];

  const int lane = threadIdx.x & 63, a = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar: LDS bases, row side
  const int side = w / WR;                                 // 0: row I, 1: row I+1
  const int brow = pairs[2 * pr + side];                   // -1: the pair has one row
  const BrowInfo b0 = load_info(info, pairs[2 * pr]);
  const int Jend = pairs[2 * pr + 1] >= 0 ? b0.I + 1 : b0.I;  // last key block of the sweep
  const bool mine = brow >= 0;
  const BrowInfo bi = mine ? load_info(info, brow) : b0;
  const int rows = mine ? min(B, bi.n - bi.I * B) : 0;
  const bool partial = rows < B;
  const int q0 = 32 * (w % WR);                            // first query of this wave in its row
  const unsigned char* Kh = reinterpret_cast<const unsigned char*>(hd.k + (size_t)b0.seq0 * hd.k_stride);
  float2* zrow = STATS ? zbuf + ((size_t)h * n_causal + (mine ? coff[brow] : 0)) * B : nullptr;

  Frag<T, D> qf[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qr = q0 + 16 * qt + c;
    qf[qt].load(hd.q + (size_t)(bi.tok0 + qr) * hd.q_stride, qr < rows, a);
  }

  // key tiles: registers -> LDS, fetched two blocks ahead (LDS double buffered)
  // DMA load of key block J into LDS buffer buf: each wave fills NDMA consecutive KiB; lane l of
  // a load writes bytes 16 l .. 16 l + 15 of its KiB, i.e. chunk position p of row r, and so
  // fetches chunk p ^ kswz(r) of key J B + r (clamped into the sequence: keys past its end are
  // masked wherever they are read)
  // Each lane's source offset within a block of keys is the same for every block; only the
  // block base (uniform) changes.  The sequence's last key block is the only one that can run
  // past its end; its clamped offsets (rows past the end read the last key) are computed here
  // once, so a block's DMA only selects between two offsets instead of clamping every load.
  const int Jlast = (b0.n - 1) / B;
  uint32_t dma_off[DMA ? NDMA : 1], dma_off_last[DMA ? NDMA : 1];
  if constexpr (DMA) {
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
      const int byte = (w * NDMA + u) * 1024 + lane * 16;
      const int r = byte / (D * 2), p = (byte % (D * 2)) / 16;
      dma_off[u] = (uint32_t)(r * hd.k_stride * 2 + (p ^ kswz<D>(r)) * 16);
      const int over = Jlast * B + r - (b0.n - 1);
      dma_off_last[u] = over > 0 ? dma_off[u] - (uint32_t)over * (uint32_t)(hd.k_stride * 2) : dma_off[u];
    }
  }
  auto dma_k = [&](int J, int buf) {
    if constexpr (DMA) {
      const MF_GLOBAL unsigned char* kb = (const MF_GLOBAL unsigned char*)Kh + (size_t)J * B * hd.k_stride * 2;
      const bool last = J == Jlast;
#pragma unroll
      for (int u = 0; u < NDMA; ++u) {
        const int kib = w * NDMA + u;
        const uint32_t off = last ? dma_off_last[u] : dma_off[u];
        __builtin_amdgcn_global_load_lds(kb + off, (__attribute__((address_space(3))) void*)&s_k[buf][kib * 1024], 16, 0, 0);
      }
    }
  };
  auto dma_wait = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0): the DMA has landed
  // the same with the QT statistics stores issued after the DMA still allowed in flight
  // (vector-memory operations complete in issue order, so the older DMA has landed)
  static_assert(QT == 2, "the wait below counts QT stores");
  auto dma_wait_but_stores = [] { __builtin_amdgcn_s_waitcnt(0x0F72); };   // vmcnt(2)
  auto fetch_k = [&](v4u (&kst)[CPT], int J) {
    if constexpr (DMA) return;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int piece = threadIdx.x + u * NTHR;
      const int row = piece / CPR, col = piece % CPR;
      const int key = J * B + row;
      kst[u] = key < b0.n ? ld16(Kh + (size_t)key * hd.k_stride * sizeof(T) + col * 16) : zero_u4();
    }
  };
  auto stage_k = [&](const v4u (&kst)[CPT], int buf) {
    if constexpr (DMA) return;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int piece = threadIdx.x + u * NTHR;
      *reinterpret_cast<v4u*>(&s_k[buf][(piece / CPR) * ROWB + (piece % CPR) * 16]) = kst[u];
    }
  };

  // running base-2 logsumexp of this lane's queries (every row a of the wave holds the same ones)
  float m_run[QT];
  double l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = kNegInf;
    l_run[qt] = 0.0;
  }
  // fused prefill: output accumulators O^T (d 16 dt + 4 a + i, query c), scaled like the running
  // sum (relative to m_run), probabilities entering the fp16 MFMA scaled by 2^15
  constexpr int NDT = D / 16, NCH = B / 32;
  v4f acc[ATTN ? QT : 1][ATTN ? NDT : 1];
  if constexpr (ATTN) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] = zero4();
  }
  const int kbrow0 = pairs[2 * pr] - b0.I;                // block row holding key block 0
  // bf16 attention: each block's prepared V tile (one KV head, fp16 operand records) is staged in
  // LDS by DMA once per workgroup beside the keys, instead of every wave loading it
  constexpr bool VLDS = ATTN && DMA;
  constexpr int VT = (D / 16) * (B / 32) * 1024;          // bytes of one block's V tile
  constexpr int NVDMA = VLDS ? VT / 1024 / (NTHR / 64) : 1;
  __shared__ __attribute__((aligned(16))) unsigned char s_v[VLDS ? 2 : 1][VLDS ? VT : 16];
  auto dma_v = [&](int J, int buf) {
    if constexpr (VLDS) {
      const MF_GLOBAL unsigned char* vsrc = (const MF_GLOBAL unsigned char*)(
          ao.vfrag + (((size_t)hd.vhead * n_brow + kbrow0 + J) * (B / 32)) * (D / 16) * 512);
#pragma unroll
      for (int u = 0; u < NVDMA; ++u) {
        const int kib = w * NVDMA + u;
        __builtin_amdgcn_global_load_lds(vsrc + kib * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void*)&s_v[buf][kib * 1024], 16, 0, 0);
      }
    }
  };
  v4u kst[CPT];
  // A block's statistics are stored during the next block, right after that block's key DMA, so
  // the wait for the DMA at its end need not cover them.
  float2 zpend[QT];
  int Jpend = -1;                                         // block whose statistics are pending
  // block(J, Tag<true>): this wave computes block J; Tag<false>: it only issues the loads and
  // stores.  The two kinds run in separate loops (every block a wave computes comes first), so no
  // path into the LDS reads of a computed block passes an LDS DMA still in flight.
  auto block = [&](int J, auto kind) {
    constexpr bool COMPUTE = decltype(kind)::value;
    if (J + 1 <= Jend) fetch_k(kst, J + 1);
    const bool stored = STATS && Jpend >= 0;
    // The next block's key (and V) tile DMA, into the buffers last read in block J - 1, then the
    // previous block's statistics.  The DMA is issued after this block's score reads of the keys:
    // the compiler cannot tell the two LDS buffers apart and makes every LDS read wait for all LDS
    // DMA in flight, so a DMA issued before the score products would be waited for at once, with
    // nothing to hide its latency; issued after them, it lands during the exponentials (the
    // attention half's V reads, which follow, wait for what is left of it).
    // Every lane group stores (the four hold the same values): the stores stay unconditional, so
    // the end-of-block wait that lets them stay in flight is known to cover the DMA on every path.
    auto issue = [&] {
      if (J + 1 <= Jend) {
        dma_k(J + 1, (J + 1) & 1);
        dma_v(J + 1, (J + 1) & 1);
      }
      if (stored) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) zrow[(size_t)Jpend * B + q0 + 16 * qt + c] = zpend[qt];
        Jpend = -1;
      }
    };
    if constexpr (COMPUTE) {
      const unsigned char* kt = s_k[J & 1];
      v4f s[QT][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag<T, D> kf;
        if constexpr (DMA) load_lds_frag_swz<D>(kf, kt, 16 * mt + c, a);
        else load_lds_frag<D>(kf, kt + (16 * mt + c) * ROWB, a);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt][mt] = dot_tile<D>(kf, qf[qt], zero4());
      }
      issue();
      // only the diagonal block and blocks of a partial row need the causal / length mask
      const bool masked = J == bi.I || partial;
      v8h pop[ATTN ? QT : 1][NCH];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int qr = q0 + 16 * qt + c;
        const int qloc = bi.I * B + qr;
        float2 zr;
        bool done = false;
        if constexpr (!ATTN) {
          // past the first block, an unmasked block is summed against the running maximum
          // instead of its own: z = sum_j 2^(s_j c - m_run), stored with reference m_run, and the
          // running sum just adds it.  Should the block's scores rise far above m_run (z reaching
          // 2^64 in some row), the whole wave redoes it with the block maximum below.  A finite
          // m_run is guaranteed here: block 0 of a row always holds a visible key.
          if (!masked && J > 0) {
            float z = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) z += fast_exp2(fmaf(s[qt][mt][i], scale2, -m_run[qt]));
            z = xrow_sum(z);
            done = __builtin_amdgcn_ballot_w64(!(z < 0x1p64f)) == 0;
            if (done) {
              zr = make_float2(z, m_run[qt]);
              l_run[qt] += (double)z;
            }
          }
        }
        if constexpr (ATTN) {
          // statistics against the new running maximum; s holds the block's fp16-scaled
          // probabilities, and the output is rescaled to the new maximum
          zr = masked ? block_stats_run<MT, true>(s[qt], J * B + 4 * a - qloc, qr < rows, scale2, m_run[qt])
                      : block_stats_run<MT, false>(s[qt], 0, true, scale2, m_run[qt]);
          if (STATS) zpend[qt] = zr;
          float alpha = 1.f;
          if (zr.x > 0.f) {
            if (zr.y != m_run[qt]) alpha = fast_exp2(m_run[qt] - zr.y);   // 0 on a row's first block
            l_run[qt] = l_run[qt] * (double)alpha + (double)zr.x;
            m_run[qt] = zr.y;
          }
          // past the first blocks of a row its running maximum rarely moves: the wave skips the
          // rescale when every alpha is exactly 1
          if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[qt][dt][i] *= alpha;
          }
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const f2 v2 = {s[qt][2 * ch + (e >> 2)][e & 3], s[qt][2 * ch + ((e + 1) >> 2)][(e + 1) & 3]};
              pk[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, h2));
            }
            pop[qt][ch] = as_v8h(v4u{pk[0], pk[1], pk[2], pk[3]});
          }
        } else {
          if (!done) {
            zr = masked ? block_stats<MT, true>(s[qt], J * B + 4 * a - qloc, qr < rows, scale2)
                        : block_stats<MT, false>(s[qt], 0, true, scale2);
          }
          if (STATS) zpend[qt] = zr;
          if (!done && zr.x > 0.f) {
            const float mn = __builtin_fmaxf(m_run[qt], zr.y);
            l_run[qt] = l_run[qt] * (double)fast_exp2(m_run[qt] - mn) + (double)zr.x * (double)fast_exp2(zr.y - mn);
            m_run[qt] = mn;
          }
        }
      }
      if (STATS) Jpend = J;
      if constexpr (ATTN) {
        // P.V on the fp16 MFMA; each V operand tile serves both query tiles
        const uint16_t* vb = ao.vfrag + ((((size_t)hd.vhead * n_brow + kbrow0 + J) * NCH) * NDT) * 512 + lane * 8;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const v8h vop = VLDS ? as_v8h(*reinterpret_cast<const v4u*>(&s_v[J & 1][((ch * NDT + dt) * 64 + lane) * 16]))
                                 : as_v8h(ld16(vb + (ch * NDT + dt) * 512));
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma_f16(vop, pop[qt][ch], acc[qt][dt]);
          }
      }
    } else {
      issue();
    }
    if (J + 1 <= Jend) stage_k(kst, (J + 1) & 1);
    if (DMA) {
      if (stored) dma_wait_but_stores();
      else dma_wait();
    }
    lds_barrier();
  };
  fetch_k(kst, 0);
  stage_k(kst, 0);
  dma_k(0, 0);
  dma_v(0, 0);
  if (DMA) dma_wait();
  __syncthreads();
  const int Jc = mine ? bi.I : -1;                         // last block this wave computes
  int J = 0;
  for (; J <= Jc; ++J) block(J, BoolTag<true>{});
  for (; J <= Jend; ++J) block(J, BoolTag<false>{});
  if (STATS && Jpend >= 0 && a == 0) {                     // the last block's statistics
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) zrow[(size_t)Jpend * B + q0 + 16 * qt + c] = zpend[qt];
  }
  // ---- row logsumexp, then block masses (one coalesced read per block and wave) ------------
  if (STATS && mine && a == 0) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int qr = q0 + 16 * qt + c;
      const float v = (float)((double)m_run[qt] + log2(l_run[qt]));
      s_lse[side][qr] = v;
      if (qr < rows) lse2[(size_t)h * T_tot + bi.tok0 + qr] = v;
    }
  }
  if constexpr (ATTN) {
    if (mine) {
      const float unscale = ldexpf(1.f, -15 - ao.vexps[hd.vhead]);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int qr = q0 + 16 * qt + c;
        if (qr >= rows) continue;
        const float inv = unscale / (float)l_run[qt];
        float* orow = hd.o + (size_t)(bi.tok0 + qr) * hd.o_stride;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * a + i] = acc[qt][dt][i] * inv;
      }
    }
  }
  if constexpr (!STATS) return;
  __syncthreads();                                         // every wave reaches it
  if (!mine) return;
  float* out = Mh + ((size_t)h * n_brow + brow) * nb_max;
  const float lq = lane < rows ? s_lse[side][lane] : 0.f;
  for (int J = w % WR; J <= bi.I; J += WR) {
    const float2 e = lane < B ? zrow[(size_t)J * B + lane] : make_float2(0.f, kNegInf);
    const double v = (lane < rows && e.y > kNegInf) ? (double)e.x * (double)fast_exp2(e.y - lq) : 0.0;
    const double t = wave_sum_f64(v);
    if (lane == 0) out[J] = (float)t;
  }
}

}  // namespace mf
