// Compression of one sender layer's causal softmax map into the block-sparse store.
//
// [MapFlow开源, section 只存重要的:块稀疏压缩] (aitest123.com) and [Reuses Attention, first
// component] (roboind.com): the map is cut into regular 2-D blocks, block-level statistics are
// computed first, then the high-mass blocks are chosen by cumulative attention probability and
// stored; the dense L x L map is never assembled.
//
// Kernels, in launch order:
//   k_stats        one score pass per (block row, sender head): per (query, key block) the block
//                  maximum and scaled sum, from which the row logsumexp and the per-block mass
//                  of exp(s - lse) follow exactly
//   k_head_reduce  head-summed block masses in fp64, fixed head order
//   k_select       per block row: forced sink + diagonal, then descending mass (ties: lower
//                  column) until the kept mass reaches tau * H_s * rows
//   k_scan         counts -> block_ptr, kept-block total
//   k_emit         ascending kept columns per block row
//   k_gather       recompute kept tiles for 8 sender heads, store bf16 probs and per-chunk row sums
//   k_rowmass      kept row mass = sum of the gather's per-chunk row sums, in column order
// Scores s = q.k / sqrt(d) are formed by MFMA (bf16 inputs: 16x16x32 bf16; fp32 inputs:
// 16x16x4 f32) with fp32 accumulation; exponentials use base 2 with log2(e) folded into the
// scale.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "sweep.h"

namespace mf {

// Work item of the statistics grid: head-major, so the key rows of the few heads in flight stay
// cache resident.  With a multiple of 8 heads, head h runs on XCD h mod 8 (workgroup b runs on
// XCD b mod 8), so the workgroups in flight on one XCD sweep the keys of one head and share its
// L2.
__device__ __forceinline__ void stats_item(int H_s, int n_pair, int& h, int& pr) {
  if ((H_s & 7) == 0) {
    const int q = blockIdx.x >> 3;
    h = (q / n_pair) * 8 + (blockIdx.x & 7);
    pr = q % n_pair;
  } else {
    h = blockIdx.x / n_pair;
    pr = blockIdx.x % n_pair;
  }
}

template <typename T, int B, int D>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(4))) void k_stats(
    const T* __restrict__ Q, const T* __restrict__ K, int H_s, int64_t T_tot, const int32_t* __restrict__ info,
    const int32_t* __restrict__ pairs, int n_pair, const int32_t* __restrict__ coff, int64_t n_causal, int n_brow,
    int nb_max, float scale2, float2* __restrict__ zbuf, float* __restrict__ lse2, float* __restrict__ Mh) {
  int h, pr;
  stats_item(H_s, n_pair, h, pr);
  const SweepHead<T> hd{Q + (size_t)h * T_tot * D, D, K + (size_t)h * T_tot * D, D, h, nullptr, 0};
  sweep_body<T, B, D, false, true>(hd, h, pr, T_tot, info, pairs, coff, n_causal, n_brow, nb_max, scale2, zbuf,
                                   lse2, Mh, AttnOut{nullptr, nullptr});
}

// The fused prefill: the same statistics (bit for bit: the same code computes them) plus the
// sender's own causal attention output [T][H_s][D] from the same scores.
template <typename T, int B, int D>
__global__ __launch_bounds__(B * 4) void k_prefill(
    const T* __restrict__ Q, const T* __restrict__ K, int H_s, int64_t T_tot, const int32_t* __restrict__ info,
    const int32_t* __restrict__ pairs, int n_pair, const int32_t* __restrict__ coff, int64_t n_causal, int n_brow,
    int nb_max, float scale2, float2* __restrict__ zbuf, float* __restrict__ lse2, float* __restrict__ Mh,
    AttnOut ao, float* __restrict__ O) {
  int h, pr;
  stats_item(H_s, n_pair, h, pr);
  const SweepHead<T> hd{Q + (size_t)h * T_tot * D, D, K + (size_t)h * T_tot * D, D, h, O + (size_t)h * D,
                        (int64_t)H_s * D};
  sweep_body<T, B, D, true, true>(hd, h, pr, T_tot, info, pairs, coff, n_causal, n_brow, nb_max, scale2, zbuf,
                                  lse2, Mh, ao);
}

// ------------------------------------------------------------------------------------------
__global__ void k_head_reduce(const float* __restrict__ Mh, int H_s, int n_brow, int nb_max,
                              const int32_t* __restrict__ info, double* __restrict__ M) {
  const int brow = blockIdx.x;
  const int I = info[4 * brow + 3];
  for (int J = threadIdx.x; J <= I; J += blockDim.x) {
    double s = 0.0;
    for (int h = 0; h < H_s; ++h) s += (double)Mh[((size_t)h * n_brow + brow) * nb_max + J];
    M[(size_t)brow * nb_max + J] = s;
  }
}

// ------------------------------------------------------------------------------------------
// k_select: one workgroup per block row.  Non-forced columns are sorted in LDS (bitonic, key =
// mass descending then column ascending), then one lane walks them in order, exactly as the
// definition: stop as soon as the cumulative mass (forced blocks included) reaches the target.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bool sel_before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// One block row's selection over masses Mrow[0..I] (total mass heads * rows): forced sink and
// diagonal, then a bitonic sort of (-mass, column) in LDS and a sequential walk by one lane.
template <typename MT>
__device__ __forceinline__ void select_row(const MT* __restrict__ Mrow, int I, int rows, int heads, double tau,
                                           uint8_t* __restrict__ frow, int32_t* __restrict__ count_out,
                                           unsigned char* sm_raw) {
  const int n = I + 1;
  if (tau >= 1.0) {
    for (int J = threadIdx.x; J < n; J += blockDim.x) frow[J] = 1;
    if (threadIdx.x == 0 && count_out) *count_out = n;
    return;
  }
  int N = 1;
  while (N < n) N <<= 1;
  double* key = reinterpret_cast<double*>(sm_raw);
  int* idx = reinterpret_cast<int*>(sm_raw + sizeof(double) * N);
  for (int t = threadIdx.x; t < N; t += blockDim.x) {
    const bool real = t < n && t != 0 && t != I;
    key[t] = real ? (double)Mrow[t] : -1.0;   // masses are >= 0; -1 marks forced / padding slots
    idx[t] = t;
    if (t < n) frow[t] = (t == 0 || t == I) ? 1 : 0;
  }
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < N; t += blockDim.x) {
        const int u = t ^ j;
        if (u > t) {
          const bool up = (t & k) == 0;  // this pair must end in "before" order
          const bool tb = sel_before(key[t], idx[t], key[u], idx[u]);
          if (tb != up) {
            const double kt = key[t];
            key[t] = key[u];
            key[u] = kt;
            const int it = idx[t];
            idx[t] = idx[u];
            idx[u] = it;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    double c = (double)Mrow[0];
    int cnt = 1;
    if (I > 0) {
      c += (double)Mrow[I];
      cnt = 2;
    }
    const double target = tau * (double)(heads * rows);
    for (int t = 0; t < N; ++t) {
      if (key[t] < 0.0 || c >= target) break;
      frow[idx[t]] = 1;
      c += key[t];
      ++cnt;
    }
    if (count_out) *count_out = cnt;
  }
}

__global__ __launch_bounds__(256) void k_select(const double* __restrict__ M,
                                                const int32_t* __restrict__ info, int nb_max,
                                                int H_s, int B, double tau,
                                                const uint8_t* __restrict__ active,
                                                uint8_t* __restrict__ flags,
                                                int32_t* __restrict__ counts) {
  extern __shared__ unsigned char sm_raw[];
  const int brow = blockIdx.x;
  if (active != nullptr && !active[brow]) {        // a row outside the compressed range keeps nothing
    if (threadIdx.x == 0) counts[brow] = 0;
    return;
  }
  const BrowInfo bi = load_info(info, brow);
  const int rows = min(B, bi.n - bi.I * B);
  select_row<double>(M + (size_t)brow * nb_max, bi.I, rows, H_s, tau, flags + (size_t)brow * nb_max, counts + brow,
                     sm_raw);
}

// Selection per sender head (the per-head variant): head h = blockIdx.y selects from its own
// block masses with total mass rows; the kept flags of every head are then united by k_union.
__global__ __launch_bounds__(256) void k_select_heads(const float* __restrict__ Mh,
                                                      const int32_t* __restrict__ info, int n_brow,
                                                      int nb_max, int B, double tau,
                                                      const uint8_t* __restrict__ active,
                                                      uint8_t* __restrict__ hflags) {
  extern __shared__ unsigned char sm_raw[];
  const int brow = blockIdx.x, h = blockIdx.y;
  if (active != nullptr && !active[brow]) return;
  const BrowInfo bi = load_info(info, brow);
  const int rows = min(B, bi.n - bi.I * B);
  const size_t off = ((size_t)h * n_brow + brow) * nb_max;
  select_row<float>(Mh + off, bi.I, rows, 1, tau, hflags + off, nullptr, sm_raw);
}

// Kept flags of a block row = union over the heads' own selections; counts for the scan.
__global__ __launch_bounds__(256) void k_union(const uint8_t* __restrict__ hflags, int H_s, int n_brow,
                                               int nb_max, const int32_t* __restrict__ info,
                                               const uint8_t* __restrict__ active,
                                               uint8_t* __restrict__ flags, int32_t* __restrict__ counts) {
  __shared__ int part[4];
  const int brow = blockIdx.x;
  if (active != nullptr && !active[brow]) {
    if (threadIdx.x == 0) counts[brow] = 0;
    return;
  }
  const int I = info[4 * brow + 3];
  int cnt = 0;
  for (int J = threadIdx.x; J <= I; J += blockDim.x) {
    uint8_t f = 0;
    for (int h = 0; h < H_s; ++h) f |= hflags[((size_t)h * n_brow + brow) * nb_max + J];
    flags[(size_t)brow * nb_max + J] = f ? 1 : 0;
    cnt += f ? 1 : 0;
  }
  cnt = (int)wave_sum((float)cnt);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) counts[brow] = part[0] + part[1] + part[2] + part[3];
}

// Per-head normalisation (variant): each head's kept mass of every query row, from the block
// statistics (z, r) of its kept blocks, folded into that head's logsumexp for the gather:
// lse2n = lse2 + log2(sum over kept J of z_iJ 2^(r_iJ - lse2)).
__global__ void k_keptnorm(const float2* __restrict__ zbuf, const float* __restrict__ lse2,
                           const int32_t* __restrict__ block_ptr, const int32_t* __restrict__ block_idx,
                           const int32_t* __restrict__ info, const int32_t* __restrict__ coff,
                           const int32_t* __restrict__ counters, const uint8_t* __restrict__ active,
                           const uint8_t* __restrict__ hflags, int n_brow, int nb_max, int B, int64_t n_causal,
                           int64_t T_tot, int64_t capacity, float* __restrict__ lse2n) {
  const int brow = blockIdx.x, h = blockIdx.y, r = threadIdx.x;
  if (active != nullptr && !active[brow]) return;
  const BrowInfo bi = load_info(info, brow);
  const int rows = min(B, bi.n - bi.I * B);
  if (r >= rows) return;
  const int64_t nnzb = min((int64_t)counters[0], capacity);
  const int64_t lo = min((int64_t)block_ptr[brow], nnzb), hi = min((int64_t)block_ptr[brow + 1], nnzb);
  const float2* zrow = zbuf + ((size_t)h * n_causal + coff[brow]) * B;
  const float l = lse2[(size_t)h * T_tot + bi.tok0 + r];
  double s = 0.0;
  for (int64_t t = lo; t < hi; ++t) {
    const int J = block_idx[t];
    if (hflags != nullptr && !hflags[((size_t)h * n_brow + brow) * nb_max + J]) continue;
    const float2 e = zrow[(size_t)J * B + r];
    if (e.y > kNegInf) s += (double)e.x * (double)fast_exp2(e.y - l);
  }
  lse2n[(size_t)h * T_tot + bi.tok0 + r] = s > 0.0 ? (float)((double)l + log2(s)) : l;
}

// ------------------------------------------------------------------------------------------
// k_scan: exclusive scan of the per-row counts (single workgroup).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ counts, int n_brow,
                                               int64_t capacity, int32_t* __restrict__ block_ptr,
                                               int32_t* __restrict__ counters) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  const int chunk = (n_brow + 1023) / 1024;
  const int lo = min(n_brow, t * chunk), hi = min(n_brow, lo + chunk);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += counts[i];
  sums[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int run = sums[t] - s;  // exclusive prefix of this thread's chunk
  for (int i = lo; i < hi; ++i) {
    block_ptr[i] = run;
    run += counts[i];
  }
  if (t == 1023) {
    const int total = sums[1023];
    block_ptr[n_brow] = total;
    counters[0] = total;
    counters[1] = (int64_t)total > capacity ? 1 : 0;
  }
}

// ------------------------------------------------------------------------------------------
// k_emit: kept columns of one block row in ascending order (wave ballots + workgroup prefix).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(const uint8_t* __restrict__ flags,
                                              const int32_t* __restrict__ block_ptr,
                                              const int32_t* __restrict__ info, int nb_max,
                                              int64_t capacity, const uint8_t* __restrict__ active,
                                              int32_t* __restrict__ block_idx,
                                              int32_t* __restrict__ block_row) {
  __shared__ int wtot[4];
  const int brow = blockIdx.x;
  if (active != nullptr && !active[brow]) return;   // its flags are stale scratch
  const int I = info[4 * brow + 3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint8_t* frow = flags + (size_t)brow * nb_max;
  int run = block_ptr[brow];
  for (int base = 0; base <= I; base += 256) {
    const int J = base + threadIdx.x;
    const bool f = J <= I && frow[J];
    const unsigned long long mask = __ballot(f);
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[w] = __popcll(mask);
    __syncthreads();
    int off = 0;
    for (int r = 0; r < w; ++r) off += wtot[r];
    int tot = 0;
    for (int r = 0; r < 4; ++r) tot += wtot[r];
    const int64_t pos = (int64_t)run + off + rank;
    if (f && pos < capacity) {
      block_idx[pos] = J;
      block_row[pos] = brow;
    }
    run += tot;
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// k_gather: one workgroup per (chunk of kGatherChunk kept blocks of a block row, group of 8 sender
// heads),
// 8 waves; wave w owns sender head 8*hg + w and keeps that head's query rows of the block row in
// registers.  Work items are ordered chunk-major, so the workgroups in flight share one range of
// key blocks in L2.  Per kept block of the chunk, in column order, and 16-key slice:
//   * the slice's key operands are loaded B/16 - 1 slices ahead from the key tiles written by
//     k_ktile, already in MFMA fragment layout: each load instruction reads 1 KiB of contiguous
//     memory (loading the fragments from the plain key rows would touch 16 rows per instruction
//     and make the vector L1 the bottleneck);
//   * scores are formed transposed on MFMA (lane (a, c): keys 16 nt + 4 a + i of row c) and
//     turned into bf16 probabilities exp(s - lse); the stored values of two slices, packed, are
//     summed per row on MFMA against an all-ones operand (the row sums of the stored values);
//   * the values are written into an LDS tile laid out like the stored 16-byte records of 8
//     heads per (row, column), with key positions and head slots permuted by the row so that one
//     wave's 2-byte writes hit distinct banks;
// once all 8 waves have written their head, the tile is streamed to HBM with the rotation undone,
// with non-temporal stores spread over the next block's slices, each part issued right after
// that slice's key loads (LDS double buffered where it fits: one barrier per block).
// The causal / partial-row mask is evaluated only on blocks that need it.
// ------------------------------------------------------------------------------------------
// Key operands in MFMA fragment layout.  For sender head h, block row kb (used as key block),
// 16-key slice nt, fragment element k and lane l = (a, c): element k of Frag<T, D> for key
// 16 nt + c of that block, i.e. K[h][key][32 k + 8 a .. +8] (bf16) or K[h][key][4 k + a] (fp32).
// Every (slice, element) is one contiguous run over the 64 lanes, so the gather loads its
// operands with fully coalesced loads straight into registers; keys beyond the sequence are 0.
template <typename T, int D>
struct KTile {
  static constexpr int kElems = Frag<T, D>::N;                                  // per lane and slice
  static constexpr int kElemBytes = (int)sizeof(Frag<T, D>::v[0]);
  static constexpr int kSliceBytes = kElems * 64 * kElemBytes;                  // = 16 keys x D
};

template <typename T, int B, int D>
__global__ __launch_bounds__(256) void k_ktile(const T* __restrict__ K, int64_t T_tot, int n_brow,
                                               const int32_t* __restrict__ info,
                                               unsigned char* __restrict__ ktile) {
  using KT = KTile<T, D>;
  constexpr int NT = B / 16;
  constexpr int PER = NT * KT::kElems * 64;                                     // elements per (h, kb)
  const int kb = blockIdx.x, h = blockIdx.y;
  const BrowInfo bi = load_info(info, kb);
  unsigned char* dst = ktile + ((size_t)h * n_brow + kb) * NT * KT::kSliceBytes;
  for (int e = threadIdx.x; e < PER; e += 256) {
    const int lane = e & 63, k = (e >> 6) % KT::kElems, nt = (e >> 6) / KT::kElems;
    const int a = lane >> 4, c = lane & 15;
    const int key = bi.I * B + 16 * nt + c;
    const T* row = K + ((size_t)h * T_tot + bi.seq0 + key) * D;
    if constexpr (sizeof(T) == 2) {
      const v4u x = key < bi.n ? ld16(row + 32 * k + 8 * a) : zero_u4();
      *reinterpret_cast<v4u*>(dst + (size_t)e * 16) = x;
    } else {
      const float x = key < bi.n ? row[4 * k + a] : 0.f;
      *reinterpret_cast<float*>(dst + (size_t)e * 4) = x;
    }
  }
}

template <int D>
__device__ __forceinline__ void ktile_load(Frag<uint16_t, D>& f, const unsigned char* slice, int lane) {
#pragma unroll
  for (int k = 0; k < Frag<uint16_t, D>::N; ++k) f.v[k] = as_v8s(ld16(slice + (k * 64 + lane) * 16));
}
template <int D>
__device__ __forceinline__ void ktile_load(Frag<float, D>& f, const unsigned char* slice, int lane) {
#pragma unroll
  for (int k = 0; k < Frag<float, D>::N; ++k) f.v[k] = *reinterpret_cast<const float*>(slice + (k * 64 + lane) * 4);
}

// LDS record tile of one kept block: for every (row r, key k) a 16-byte record of the 8 heads of
// the group, bf16.  Wave w (head 8 hg + w) forms its scores transposed, so lane (a, c) holds keys
// 16 nt + 4 a + i of row 16 mt + c; its 2-byte writes would all hit the same four banks (the 16
// rows are 1 KiB apart), so two functions of c = r mod 16 spread them:
//   * the record of key k sits at position k ^ kv(c) of its row (kv flips the key's low 2 bits),
//   * the head slots of the record are rotated by kg(c) dwords (head w at halfword (w + 2 kg) mod 8);
// (kv, kg) takes all 16 values as c does, so one wave's writes of one i hit 64 distinct banks.
// On the way out a wave reads one row (B = 64) or two rows whose kg agrees (B = 32), so the
// rotation is uniform there and the reads are 16-byte, conflict-free.
__device__ __forceinline__ int rec_xor(int c) { return (c & 1) | ((c >> 3) << 1); }
__device__ __forceinline__ int rec_rot(int c) { return (c >> 1) & 3; }

// Stream part q of NQ of a finished record tile (B x B records of 16 bytes) to HBM in (row, key)
// order with the head-slot rotation undone.  Each thread handles contiguous 16-byte pieces.
template <int B>
__device__ __forceinline__ void stream_tile(const unsigned char* tile, unsigned char* dst, int q, int NQ,
                                            int w, int lane) {
  constexpr int PIECES = B * B / 512;              // pieces per thread per tile
  const int per = PIECES / NQ;
  if constexpr (B == 64) {
    // Piece u0 of wave w is row r = 16 (w / 2) + 2 (u0 mod 4) + 8 (u0 / 4) + (w mod 2), record
    // k = lane.  The 8 waves x 8 pieces cover the 64 rows once, each wave instruction still
    // stores one whole row (1 KiB), and the row's head-slot rotation rec_rot(r mod 16) = u0 mod 4
    // is known at compile time: no branch per piece, and the reads of a part can be issued
    // together before their wait.
#pragma unroll
    for (int u0 = 0; u0 < PIECES; ++u0) {
      if (u0 / per != q) continue;
      const int rr = 2 * (u0 & 3) + 8 * (u0 >> 2) + (w & 1);    // r mod 16
      const int r = 16 * (w >> 1) + rr;
      const v4u x = *reinterpret_cast<const v4u*>(tile + (r * B + (lane ^ rec_xor(rr))) * 16);
      v4u y;
      if ((u0 & 3) == 0) y = x;
      else if ((u0 & 3) == 1) y = v4u{x[1], x[2], x[3], x[0]};
      else if ((u0 & 3) == 2) y = v4u{x[2], x[3], x[0], x[1]};
      else y = v4u{x[3], x[0], x[1], x[2]};
      __builtin_nontemporal_store(y, reinterpret_cast<v4u*>(dst + ((size_t)r * B + lane) * 16));
    }
    return;
  }
#pragma unroll
  for (int u0 = 0; u0 < PIECES; ++u0) {
    if (u0 / per != q) continue;
    const int piece = 64 * w + lane + u0 * 512;
    const int r = piece / B, k = piece % B;
    const int rot = rec_rot((64 * w + u0 * 512) / B % 16);   // uniform over the wave
    const v4u x = *reinterpret_cast<const v4u*>(tile + (r * B + (k ^ rec_xor(r % 16))) * 16);
    v4u y;
    if (rot == 0) y = x;
    else if (rot == 1) y = v4u{x[1], x[2], x[3], x[0]};
    else if (rot == 2) y = v4u{x[2], x[3], x[0], x[1]};
    else y = v4u{x[3], x[0], x[1], x[2]};
    __builtin_nontemporal_store(y, reinterpret_cast<v4u*>(dst + (size_t)piece * 16));
  }
}

// One kept block for one wave: scores of the block transposed (keys x rows) on MFMA, bf16
// probabilities 2^(s c - lse2) written into the record tile, and the row sums of the stored
// values accumulated on MFMA: the packed probabilities of two key slices form the B operand
// (8 keys of row c per lane) against an all-ones A operand, so each product adds 32 keys of 16
// rows.  rsum[mt] ends with the row total of row 16 mt + c in every element.
template <typename T, int B, int D, bool HAS_PREV>
__device__ __forceinline__ void gather_block(bool MASKED, const Frag<T, D> (&qf)[B / 16], const float (&l2)[B / 16],
                                             Frag<T, D> (&kb)[B / 16], const unsigned char* ktj,
                                             const unsigned char* ktn, int J, int rows,
                                             int qdiag, float scale2, unsigned char* tile, const int (&woff)[4],
                                             int w, int lane, int a, int c, v4f (&rsum)[B / 16],
                                             const unsigned char* prev, unsigned char* prev_dst) {
  constexpr int MT = B / 16;   // 16-row tiles
  constexpr int NT = B / 16;   // 16-key slices; slice nt lives in kb[nt]
  constexpr int SB = KTile<T, D>::kSliceBytes;
  static_assert(NT % 2 == 0, "row sums pair the key slices");
  uint32_t one2 = 0x3F803F80u;                     // (1, 1) in bf16
  asm volatile("" : "+v"(one2));
  const v8s ones = as_v8s(v4u{one2, one2, one2, one2});
  uint32_t pend[MT][2];                            // packed probabilities of the even slice
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // the slice NT-1 ahead (the last of this block, or one of the next block's; past the chunk's
    // last block, this block's own slice again) into the register set slice nt-1 has finished
    // with.  Every load and store of the loop is unconditional: vector-memory operations complete
    // in issue order on one counter, and conditional ones would make the compiler's wait counts
    // conservative enough to wait for the slices prefetched ahead.
    if (nt == 0) ktile_load<D>(kb[NT - 1], ktj + (NT - 1) * SB, lane);
    else ktile_load<D>(kb[nt - 1], ktn + (nt - 1) * SB, lane);
    // a part of the previous block's tile goes out after the key loads, so no wait on a key
    // slice ever covers these stores
    if constexpr (HAS_PREV) stream_tile<B>(prev, prev_dst, nt, NT, w, lane);
    // the slice's score tiles, the MT accumulation chains interleaved step by step over the head
    // dimension so that no product waits on the one just issued
    v4f scs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) scs[mt] = zero4();
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < Frag<T, D>::N; ++k)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) scs[mt] = mfma_bf16(kb[nt].v[k], qf[mt].v[k], scs[mt]);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) scs[mt] = dot_tile<D>(kb[nt], qf[mt], zero4());
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v4f sc = scs[mt];   // keys 16 nt + 4 a + i, row 16 mt + c
      if (MASKED) {
        // diagonal / partial blocks only: invisible keys and padding rows get -inf scores
        int kq = J * B + 16 * nt + 4 * a - qdiag - 16 * mt - c;   // key (i = 0) minus query
        int rv = rows - 16 * mt - c;                               // > 0: the row exists
        asm volatile("" : "+v"(kq), "+v"(rv));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(rv > 0 && kq + i <= 0)) sc[i] = -__builtin_inff();
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sc[i], scale2, -l2[mt]));
      const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{p[0], p[1]}), b2));
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{p[2], p[3]}), b2));
      unsigned char* rec = tile + (16 * mt * B + 16 * nt) * 16;
      *reinterpret_cast<uint16_t*>(rec + woff[0]) = (uint16_t)lo;
      *reinterpret_cast<uint16_t*>(rec + woff[1]) = (uint16_t)(lo >> 16);
      *reinterpret_cast<uint16_t*>(rec + woff[2]) = (uint16_t)hi;
      *reinterpret_cast<uint16_t*>(rec + woff[3]) = (uint16_t)(hi >> 16);
      if (nt & 1)
        rsum[mt] = mfma_bf16(ones, as_v8s(v4u{pend[mt][0], pend[mt][1], lo, hi}), rsum[mt]);
      else {
        pend[mt][0] = lo;
        pend[mt][1] = hi;
      }
    }
  }
}

template <typename T, int B, int D>
struct GatherLds {
  static constexpr int kTile = B * B * 16;                               // 8-head records of a block
  static constexpr int kBufs = 2;
};

template <typename T, int B, int D, bool SELH>
__global__ __launch_bounds__(512) void k_gather(const T* __restrict__ Q, const T* __restrict__ K,
                                                int H_s, int64_t T_tot,
                                                const int32_t* __restrict__ info,
                                                const int32_t* __restrict__ order, int n_brow, int n_order,
                                                const int32_t* __restrict__ block_ptr,
                                                const int32_t* __restrict__ block_idx,
                                                const int32_t* __restrict__ counters,
                                                int64_t capacity, const float* __restrict__ lse2,
                                                float scale2, const unsigned char* __restrict__ ktile,
                                                const uint8_t* __restrict__ hflags, int nb_max,
                                                uint16_t* __restrict__ probs, double* __restrict__ part) {
  constexpr int MT = B / 16;
  constexpr int NT = B / 16;
  using L = GatherLds<T, B, D>;
  constexpr int TILE = L::kTile;
  constexpr int NBUF = L::kBufs;
  constexpr int SB = KTile<T, D>::kSliceBytes;
  constexpr int PIECES = TILE / 16 / 512;
  static_assert(PIECES >= 1 && (TILE / 16) % 512 == 0, "tile must split evenly over 512 threads");
  __shared__ __attribute__((aligned(16))) unsigned char s_out[NBUF][TILE];

  // work item (chunk k of a block row's kept list, head group, block row in the gather's order:
  // longest rows first, rows of one sequence grouped per XCD in a batch), chunk index slowest:
  // the workgroups in flight sweep the same range of key blocks, whose tiles then stay in L2 for
  // all of them.  When the head groups divide the 8 XCDs, each XCD (workgroup
  // b runs on XCD b mod 8) serves one head group, so its L2 only holds that group's key tiles.
  const int HG = (H_s + 7) >> 3;
  int p, hg, chunk;
  if ((8 % HG) == 0) {
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int nparts = 8 / HG, rp = (n_order + nparts - 1) / nparts;
    hg = xcd % HG;
    chunk = q / rp;
    p = (q % rp) * nparts + xcd / HG;
    if (p >= n_order) return;
  } else {
    p = blockIdx.x % n_order;
    hg = (blockIdx.x / n_order) % HG;
    chunk = blockIdx.x / (n_order * HG);
  }
  const int brow = order[p];
  const BrowInfo bi = load_info(info, brow);
  // the wave index is made scalar so that head-dependent choices (padding heads, masking) and the
  // tile rotation branch on the scalar unit instead of through the execution mask
  const int lane = threadIdx.x & 63, a = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = min(B, bi.n - bi.I * B);
  const int qdiag = bi.I * B;
  const int h = 8 * hg + w;
  const bool active = h < H_s;                     // padding heads write zeros
  const int64_t nnzb = min((int64_t)counters[0], capacity);
  const int64_t r0 = block_ptr[brow] + (int64_t)chunk * kGatherChunk;
  const int t0 = (int)min(r0, nnzb);
  const int t1 = (int)min(min((int64_t)block_ptr[brow + 1], r0 + kGatherChunk), nnzb);
  if (t0 >= t1) return;

  const int hq = active ? h : 0;
  // lane (a, c) handles row 16 mt + c of every 16-row tile
  Frag<T, D> qf[MT];
  float l2[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + c;
    qf[mt].load(Q + (size_t)hq * T_tot * D + (size_t)(bi.tok0 + r) * D, active && r < rows, a);
    l2[mt] = (active && r < rows) ? lse2[(size_t)hq * T_tot + bi.tok0 + r] : 0.f;
  }
  // byte offsets in the record tile of this lane's keys 4 a + i of row c (tile (0, 0)), head slot
  // of head w rotated by rec_rot(c)
  int woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    woff[i] = (c * B + 4 * a + (i ^ rec_xor(c))) * 16 + ((w + 2 * rec_rot(c)) & 7) * 2;
  // this head's key operand tiles; key block J of the sequence is block row kbrow0 + J
  const int kbrow0 = brow - bi.I;
  const unsigned char* kth = ktile + (size_t)hq * n_brow * NT * SB;
  auto kt_block = [&](int J) { return kth + (size_t)(kbrow0 + J) * NT * SB; };

  // software pipeline over the row's key slices: slice nt of a block lives in kb[nt]; the first
  // NT-1 slices of the first block are requested here, every later slice NT-1 slices ahead
  Frag<T, D> kb[NT];
  {
    const unsigned char* k0 = kt_block(block_idx[t0]);
#pragma unroll
    for (int nt = 0; nt + 1 < NT; ++nt) ktile_load<D>(kb[nt], k0 + nt * SB, lane);
  }
  double rsum_chunk = 0.0;
  // one kept block: scores, probabilities into the record tile, row sums; with HAS_PREV the
  // previous block's tile streams out meanwhile (the first block of the chunk has none)
  auto one = [&](auto has_prev, int t) {
    constexpr bool HP_ = decltype(has_prev)::value;
    const int J = block_idx[t];
    const int Jn = block_idx[min(t + 1, t1 - 1)];
    unsigned char* tile = s_out[(t - t0) % NBUF];
    v4f rsum[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rsum[mt] = zero4();
    const unsigned char* prev = s_out[(t - t0 + 1) % NBUF];
    unsigned char* prev_dst = reinterpret_cast<unsigned char*>(probs) + ((size_t)(t - 1) * HG + hg) * (size_t)TILE;
    // a head that did not select this block (per-head selection) stores zeros
    bool keep = active;
    if constexpr (SELH) keep = keep && hflags[((size_t)h * n_brow + brow) * nb_max + J];
    gather_block<T, B, D, HP_>(!keep || J == bi.I || rows < B, qf, l2, kb, kt_block(J), kt_block(Jn), J,
                               keep ? rows : 0, qdiag, scale2, tile, woff, w, lane, a, c, rsum, prev, prev_dst);
    {
      // row sums of the stored values, summed over the chunk in column order: lane (a, c) holds
      // row 16 a + c
      float v = rsum[0][0];
#pragma unroll
      for (int mt = 1; mt < MT; ++mt) v = a == mt ? rsum[mt][0] : v;
      rsum_chunk += (double)v;
    }
    // the tile is complete for streaming in the next block, and the other buffer (streamed during
    // this block) may be written again; the stores and key loads in flight stay in flight
    lds_barrier();
  };
  static_assert(NBUF == 2, "the previous block's tile streams from the other buffer");
  one(std::false_type{}, t0);
  for (int t = t0 + 1; t < t1; ++t) one(std::true_type{}, t);
  // the last block's tile
  stream_tile<B>(s_out[(t1 - 1 - t0) % NBUF],
                 reinterpret_cast<unsigned char*>(probs) + ((size_t)(t1 - 1) * HG + hg) * (size_t)TILE, 0, 1, w,
                 lane);
  // the chunk's row sums, one slot per (block row, chunk)
  const int n_chunk = (nb_max + kGatherChunk - 1) / kGatherChunk;
  if (active && a < MT) part[(((size_t)brow * n_chunk + chunk) * H_s + h) * B + 16 * a + c] = rsum_chunk;
}

// ------------------------------------------------------------------------------------------
// kept row mass: the row's chunk sums (each over up to kGatherChunk kept blocks, in column order) added in
// chunk order, fp64 throughout
__global__ void k_rowmass(const double* __restrict__ part, const int32_t* __restrict__ block_ptr,
                          const int32_t* __restrict__ info, const int32_t* __restrict__ counters,
                          int H_s, int B, int nb_max, int64_t T_tot, int64_t capacity, float* __restrict__ rkm) {
  const int brow = blockIdx.x, h = blockIdx.y, r = threadIdx.x;
  const BrowInfo bi = load_info(info, brow);
  const int rows = min(B, bi.n - bi.I * B);
  if (r >= rows) return;
  const int64_t nnzb = min((int64_t)counters[0], capacity);
  const int64_t lo = min((int64_t)block_ptr[brow], nnzb), hi = min((int64_t)block_ptr[brow + 1], nnzb);
  const int n_chunk = (nb_max + kGatherChunk - 1) / kGatherChunk;
  const int nk = (int)((hi - lo + kGatherChunk - 1) / kGatherChunk);   // chunks the gather wrote
  double s = 0.0;
  for (int k = 0; k < nk; ++k) s += part[(((size_t)brow * n_chunk + k) * H_s + h) * B + r];
  rkm[(size_t)h * T_tot + bi.tok0 + r] = (float)s;
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------

bool compress_supported(int dtype, int B, int d) {
  return (dtype == DT_F32 || dtype == DT_BF16) && (B == 32 || B == 64) && (d == 64 || d == 128);
}

template <typename T, int B, int D>
static hipError_t plan_t(const CompressArgs& a, hipStream_t s) {
  if (a.attn_out) {
    hipLaunchKernelGGL((k_prefill<T, B, D>), dim3((unsigned)a.n_pair * a.H_s), dim3(B * 4), 0, s,
                       (const T*)a.Q, (const T*)a.K, a.H_s, a.T, a.info, a.pairs, a.n_pair, a.coff,
                       a.n_causal, a.n_brow, a.nb_max, a.scale2, a.zbuf, a.lse2, a.Mh,
                       AttnOut{a.attn_vfrag, a.attn_vexps}, a.attn_out);
  } else {
    hipLaunchKernelGGL((k_stats<T, B, D>), dim3((unsigned)a.n_pair * a.H_s), dim3(B * 4), 0, s,
                       (const T*)a.Q, (const T*)a.K, a.H_s, a.T, a.info, a.pairs, a.n_pair, a.coff,
                       a.n_causal, a.n_brow, a.nb_max, a.scale2, a.zbuf, a.lse2, a.Mh);
  }
  return hipGetLastError();
}

template <typename T, int B, int D>
static hipError_t gather_t(const CompressArgs& a, hipStream_t s) {
  const int HG = (a.H_s + 7) / 8;
  if (a.capacity == 0) return hipSuccess;
  const unsigned chunks = (unsigned)((a.nb_max + kGatherChunk - 1) / kGatherChunk);
  // grid: with the XCD mapping, 8 XCDs x ceil(n_brow / (8 / HG)) block rows x chunks
  const unsigned items = (8 % HG) == 0 ? 8u * (unsigned)((a.n_order + 8 / HG - 1) / (8 / HG)) * chunks
                                       : (unsigned)a.n_order * HG * chunks;
  if (a.options & 1)
    hipLaunchKernelGGL((k_gather<T, B, D, true>), dim3(items), dim3(512), 0, s, (const T*)a.Q,
                       (const T*)a.K, a.H_s, a.T, a.info, a.order, a.n_brow, a.n_order, a.block_ptr, a.block_idx,
                       a.counters, a.capacity, (a.options & 2) ? a.lse2n : a.lse2, a.scale2,
                       (const unsigned char*)a.ktile, a.hflags, a.nb_max, a.probs, a.part);
  else
    hipLaunchKernelGGL((k_gather<T, B, D, false>), dim3(items), dim3(512), 0, s, (const T*)a.Q,
                       (const T*)a.K, a.H_s, a.T, a.info, a.order, a.n_brow, a.n_order, a.block_ptr, a.block_idx,
                       a.counters, a.capacity, (a.options & 2) ? a.lse2n : a.lse2, a.scale2,
                       (const unsigned char*)a.ktile, nullptr, a.nb_max, a.probs, a.part);
  return hipGetLastError();
}

#define MF_DISPATCH_QK(FN, A, S)                                                  \
  do {                                                                            \
    if ((A).dtype == DT_BF16) {                                                   \
      if ((A).B == 64 && (A).d == 128) return FN<uint16_t, 64, 128>(A, S);        \
      if ((A).B == 64 && (A).d == 64) return FN<uint16_t, 64, 64>(A, S);          \
      if ((A).B == 32 && (A).d == 128) return FN<uint16_t, 32, 128>(A, S);        \
      if ((A).B == 32 && (A).d == 64) return FN<uint16_t, 32, 64>(A, S);          \
    } else {                                                                      \
      if ((A).B == 64 && (A).d == 128) return FN<float, 64, 128>(A, S);           \
      if ((A).B == 64 && (A).d == 64) return FN<float, 64, 64>(A, S);             \
      if ((A).B == 32 && (A).d == 128) return FN<float, 32, 128>(A, S);           \
      if ((A).B == 32 && (A).d == 64) return FN<float, 32, 64>(A, S);             \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

template <typename T, int B, int D>
static hipError_t ktile_t(const CompressArgs& a, hipStream_t s) {
  if (a.n_brow == 0) return hipSuccess;
  hipLaunchKernelGGL((k_ktile<T, B, D>), dim3((unsigned)a.n_brow, (unsigned)a.H_s), dim3(256), 0, s,
                     (const T*)a.K, a.T, a.n_brow, a.info, (unsigned char*)a.ktile);
  return hipGetLastError();
}

static hipError_t stats_dispatch(const CompressArgs& a, hipStream_t s) { MF_DISPATCH_QK(plan_t, a, s); }
static hipError_t ktile_dispatch(const CompressArgs& a, hipStream_t s) { MF_DISPATCH_QK(ktile_t, a, s); }
static hipError_t gather_dispatch(const CompressArgs& a, hipStream_t s) { MF_DISPATCH_QK(gather_t, a, s); }

hipError_t compress_plan(const CompressArgs& a, hipStream_t s) {
  hipError_t e = ktile_dispatch(a, s);
  if (e != hipSuccess) return e;
  if ((e = stats_dispatch(a, s)) != hipSuccess) return e;
  int N = 1;
  while (N < a.nb_max) N <<= 1;
  const size_t lds = (size_t)N * (sizeof(double) + sizeof(int));
  if (a.options & 1) {                            // per-head selection, then the union
    hipLaunchKernelGGL(k_select_heads, dim3(a.n_brow, a.H_s), dim3(256), lds, s, a.Mh, a.info, a.n_brow,
                       a.nb_max, a.B, a.tau, a.active, a.hflags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_union, dim3(a.n_brow), dim3(256), 0, s, a.hflags, a.H_s, a.n_brow, a.nb_max, a.info,
                       a.active, a.flags, a.counts);
  } else {
    hipLaunchKernelGGL(k_head_reduce, dim3(a.n_brow), dim3(256), 0, s, a.Mh, a.H_s, a.n_brow,
                       a.nb_max, a.info, a.M);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_select, dim3(a.n_brow), dim3(256), lds, s, a.M, a.info, a.nb_max, a.H_s,
                       a.B, a.tau, a.active, a.flags, a.counts);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, a.counts, a.n_brow, a.capacity,
                     a.block_ptr, a.counters);
  return hipGetLastError();
}

hipError_t compress_fill(const CompressArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_emit, dim3(a.n_brow), dim3(256), 0, s, a.flags, a.block_ptr, a.info,
                     a.nb_max, a.capacity, a.active, a.block_idx, a.block_row);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.options & 2) {                            // per-head normalisation: fold kept mass into lse
    hipLaunchKernelGGL(k_keptnorm, dim3(a.n_brow, a.H_s), dim3(a.B), 0, s, a.zbuf, a.lse2, a.block_ptr,
                       a.block_idx, a.info, a.coff, a.counters, a.active, (a.options & 1) ? a.hflags : nullptr,
                       a.n_brow, a.nb_max, a.B, a.n_causal, a.T, a.capacity, a.lse2n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = gather_dispatch(a, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowmass, dim3(a.n_brow, a.H_s), dim3(a.B), 0, s, a.part, a.block_ptr,
                     a.info, a.counters, a.H_s, a.B, a.nb_max, a.T, a.capacity, a.rkm);
  return hipGetLastError();
}

}  // namespace mf
