// Compression of one sender layer's causal softmax map into the block-sparse store.
//
// [MapFlow开源, section 只存重要的:块稀疏压缩] (aitest123.com) and [Reuses Attention, first
// component] (roboind.com): the map is cut into regular 2-D blocks, block-level statistics are
// computed first, then the high-mass blocks are chosen by cumulative attention probability and
// stored; the dense L x L map is never assembled.
//
// Kernels, in launch order:
//   k_stats        two passes per (block row, sender head): pass 1 the row logsumexp (online
//                  max / sum over key blocks), pass 2 the per-block mass sum of exp(s - lse)
//   k_head_reduce  head-summed block masses in fp64, fixed head order
//   k_select       per block row: forced sink + diagonal, then descending mass (ties: lower
//                  column) until the kept mass reaches tau * H_s * rows
//   k_scan         counts -> block_ptr, kept-block total
//   k_emit         ascending kept columns per block row
//   k_gather       recompute kept tiles for 8 sender heads, store bf16 probs and per-block row sums
//   k_rowmass      kept row mass = sum over a row's kept blocks, in column order
// Scores s = q.k / sqrt(d) are formed by MFMA (bf16 inputs: 16x16x32 bf16; fp32 inputs:
// 16x16x4 f32) with fp32 accumulation; exponentials use base 2 with log2(e) folded into the
// scale.
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

// ------------------------------------------------------------------------------------------
// k_stats: row logsumexp (pass 1) and per-head block masses (pass 2) for one block row.
// Workgroup = B/16 waves; wave w owns keys 16w..16w+15 of every key block, all B queries.
// Scores are held transposed (keys x queries) so each lane accumulates statistics for its own
// query column without cross-lane traffic until the end of a pass.
// ------------------------------------------------------------------------------------------
template <typename T, int B, int D>
__global__ __launch_bounds__(B * 4) void k_stats(const T* __restrict__ Q, const T* __restrict__ K,
                                                 int H_s, int64_t T_tot,
                                                 const int32_t* __restrict__ info,
                                                 const int32_t* __restrict__ order, int n_brow,
                                                 int nb_max, float scale2, float* __restrict__ lse2,
                                                 float* __restrict__ Mh) {
  constexpr int NW = B / 16;
  constexpr int NT = B / 16;
  extern __shared__ float part[];  // [NW][nb_max]
  __shared__ float red_m[NW * 4][B];
  __shared__ float red_l[NW * 4][B];
  __shared__ float s_lse[B];

  const int h = blockIdx.x % H_s;
  const int brow = order[blockIdx.x / H_s];
  const BrowInfo bi = load_info(info, brow);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, a = lane >> 4, c = lane & 15;
  const int rows = min(B, bi.n - bi.I * B);
  const int qbase = bi.I * B;
  const T* Qh = Q + (size_t)h * T_tot * D;
  const T* Kh = K + (size_t)h * T_tot * D + (size_t)bi.seq0 * D;

  Frag<T, D> qf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int q = 16 * nt + c;
    qf[nt].load(Qh + (size_t)(bi.tok0 + q) * D, q < rows, a);
  }

  // ---- pass 1: online max / sum per query column -----------------------------------------
  float m[NT], l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { m[nt] = kNegInf; l[nt] = 0.f; }
  for (int J = 0; J <= bi.I; ++J) {
    const int key = J * B + 16 * w + c;
    Frag<T, D> kf;
    kf.load(Kh + (size_t)key * D, key < bi.n, a);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const v4f s = dot_tile<D>(kf, qf[nt], zero4());
      const int q = qbase + 16 * nt + c;
      float x[4];
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k2 = J * B + 16 * w + 4 * a + i;
        x[i] = (k2 <= q && q < bi.n) ? s[i] * scale2 : kNegInf;
        tmax = fmaxf(tmax, x[i]);
      }
      if (tmax > kNegInf) {
        const float mn = fmaxf(m[nt], tmax);
        float acc = l[nt] * fast_exp2(m[nt] - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += fast_exp2(x[i] - mn);
        m[nt] = mn;
        l[nt] = acc;
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    red_m[w * 4 + a][16 * nt + c] = m[nt];
    red_l[w * 4 + a][16 * nt + c] = l[nt];
  }
  __syncthreads();
  if (threadIdx.x < B) {
    const int q = threadIdx.x;
    float M = kNegInf;
    for (int r = 0; r < NW * 4; ++r) M = fmaxf(M, red_m[r][q]);
    float L = 0.f;
    for (int r = 0; r < NW * 4; ++r)
      if (red_m[r][q] > kNegInf) L += red_l[r][q] * fast_exp2(red_m[r][q] - M);
    const float v = M + log2f(L);
    s_lse[q] = v;
    if (q < rows) lse2[(size_t)h * T_tot + bi.tok0 + q] = v;
  }
  __syncthreads();

  // ---- pass 2: block masses ---------------------------------------------------------------
  float lq[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) lq[nt] = s_lse[16 * nt + c];
  for (int J = 0; J <= bi.I; ++J) {
    const int key = J * B + 16 * w + c;
    Frag<T, D> kf;
    kf.load(Kh + (size_t)key * D, key < bi.n, a);
    float sum = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const v4f s = dot_tile<D>(kf, qf[nt], zero4());
      const int q = qbase + 16 * nt + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k2 = J * B + 16 * w + 4 * a + i;
        if (k2 <= q && q < bi.n) sum += fast_exp2(s[i] * scale2 - lq[nt]);
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) part[w * nb_max + J] = sum;
  }
  __syncthreads();
  float* out = Mh + ((size_t)h * n_brow + brow) * nb_max;
  for (int J = threadIdx.x; J <= bi.I; J += blockDim.x) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < NW; ++r) t += part[r * nb_max + J];
    out[J] = t;
  }
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

__global__ __launch_bounds__(256) void k_select(const double* __restrict__ M,
                                                const int32_t* __restrict__ info, int nb_max,
                                                int H_s, int B, double tau,
                                                uint8_t* __restrict__ flags,
                                                int32_t* __restrict__ counts) {
  extern __shared__ unsigned char sm_raw[];
  const int brow = blockIdx.x;
  const BrowInfo bi = load_info(info, brow);
  const int I = bi.I, n = I + 1;
  const int rows = min(B, bi.n - I * B);
  const double* Mrow = M + (size_t)brow * nb_max;
  uint8_t* frow = flags + (size_t)brow * nb_max;
  if (tau >= 1.0) {
    for (int J = threadIdx.x; J < n; J += blockDim.x) frow[J] = 1;
    if (threadIdx.x == 0) counts[brow] = n;
    return;
  }
  int N = 1;
  while (N < n) N <<= 1;
  double* key = reinterpret_cast<double*>(sm_raw);
  int* idx = reinterpret_cast<int*>(sm_raw + sizeof(double) * N);
  for (int t = threadIdx.x; t < N; t += blockDim.x) {
    const bool real = t < n && t != 0 && t != I;
    key[t] = real ? Mrow[t] : -1.0;   // masses are >= 0; -1 marks forced / padding slots
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
    double c = Mrow[0];
    int cnt = 1;
    if (I > 0) {
      c += Mrow[I];
      cnt = 2;
    }
    const double target = tau * (double)(H_s * rows);
    for (int t = 0; t < N; ++t) {
      if (key[t] < 0.0 || c >= target) break;
      frow[idx[t]] = 1;
      c += key[t];
      ++cnt;
    }
    counts[brow] = cnt;
  }
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
                                              int64_t capacity, int32_t* __restrict__ block_idx,
                                              int32_t* __restrict__ block_row) {
  __shared__ int wtot[4];
  const int brow = blockIdx.x;
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
// k_gather: one workgroup per (kept block, group of 8 sender heads).  Wave w owns query rows
// 16w..16w+15; for each head the score tile is recomputed (queries x keys), exponentiated with
// the stored row logsumexp, rounded to bf16 and written as 16-byte records of 8 heads per
// (row, column), so each 16-lane group stores 256 contiguous bytes.
// ------------------------------------------------------------------------------------------
template <typename T, int B, int D>
__global__ __launch_bounds__(B * 4) void k_gather(const T* __restrict__ Q, const T* __restrict__ K,
                                                  int H_s, int64_t T_tot,
                                                  const int32_t* __restrict__ info,
                                                  const int32_t* __restrict__ block_idx,
                                                  const int32_t* __restrict__ block_row,
                                                  const int32_t* __restrict__ counters,
                                                  int64_t capacity, const float* __restrict__ lse2,
                                                  float scale2, uint16_t* __restrict__ probs,
                                                  float* __restrict__ part) {
  constexpr int NT = B / 16;
  const int HG = (H_s + 7) >> 3;
  const int64_t nblk = blockIdx.x / HG;
  const int hg = blockIdx.x - (int)(nblk * HG);
  const int64_t nnzb = min((int64_t)counters[0], capacity);
  if (nblk >= nnzb) return;
  const int brow = block_row[nblk];
  const int J = block_idx[nblk];
  const BrowInfo bi = load_info(info, brow);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, a = lane >> 4, c = lane & 15;
  const int rows = min(B, bi.n - bi.I * B);
  const int qloc0 = bi.I * B;

  v4f acc[8][NT];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) {
    const int h = hg * 8 + hh;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[hh][nt] = zero4();
    if (h >= H_s) continue;
    const T* Qh = Q + (size_t)h * T_tot * D;
    const T* Kh = K + (size_t)h * T_tot * D + (size_t)bi.seq0 * D;
    Frag<T, D> qf;
    qf.load(Qh + (size_t)(bi.tok0 + 16 * w + c) * D, 16 * w + c < rows, a);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int key = J * B + 16 * nt + c;
      Frag<T, D> kf;
      kf.load(Kh + (size_t)key * D, key < bi.n, a);
      acc[hh][nt] = dot_tile<D>(qf, kf, acc[hh][nt]);
    }
  }

  float rs[8][4];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[hh][i] = 0.f;

  uint16_t* pblk = probs + ((size_t)nblk * HG + hg) * (size_t)(B * B * 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * a + i;
    const bool vq = r < rows;
    float l2[8];
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      const int h = hg * 8 + hh;
      l2[hh] = (vq && h < H_s) ? lse2[(size_t)h * T_tot + bi.tok0 + r] : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int key = J * B + 16 * nt + c;
      const bool ok = vq && key <= qloc0 + r;
      uint32_t packed[4];
#pragma unroll
      for (int hp = 0; hp < 4; ++hp) {
        uint32_t two = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int hh = 2 * hp + e;
          const bool okh = ok && (hg * 8 + hh < H_s);
          const float p = okh ? fast_exp2(acc[hh][nt][i] * scale2 - l2[hh]) : 0.f;
          const uint16_t pb = f32_to_bf16(p);
          rs[hh][i] += bf16_to_f32(pb);
          two |= (uint32_t)pb << (16 * e);
        }
        packed[hp] = two;
      }
      st16(pblk + ((size_t)r * B + 16 * nt + c) * 8, v4u{packed[0], packed[1], packed[2], packed[3]});
    }
  }
  // row sums over the 16 lanes of each column group
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = rs[hh][i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      const int h = hg * 8 + hh;
      if (c == 0 && h < H_s) part[((size_t)nblk * H_s + h) * B + 16 * w + 4 * a + i] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
__global__ void k_rowmass(const float* __restrict__ part, const int32_t* __restrict__ block_ptr,
                          const int32_t* __restrict__ info, const int32_t* __restrict__ counters,
                          int H_s, int B, int64_t T_tot, int64_t capacity, float* __restrict__ rkm) {
  const int brow = blockIdx.x, h = blockIdx.y, r = threadIdx.x;
  const BrowInfo bi = load_info(info, brow);
  const int rows = min(B, bi.n - bi.I * B);
  if (r >= rows) return;
  const int64_t nnzb = min((int64_t)counters[0], capacity);
  const int64_t lo = min((int64_t)block_ptr[brow], nnzb), hi = min((int64_t)block_ptr[brow + 1], nnzb);
  double s = 0.0;
  for (int64_t t = lo; t < hi; ++t) s += (double)part[((size_t)t * H_s + h) * B + r];
  rkm[(size_t)h * T_tot + bi.tok0 + r] = (float)s;
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
size_t stats_lds_bytes(int B, int nb_max) { return (size_t)(B / 16) * nb_max * sizeof(float); }

bool compress_supported(int dtype, int B, int d) {
  return (dtype == DT_F32 || dtype == DT_BF16) && (B == 32 || B == 64) && (d == 64 || d == 128);
}

template <typename T, int B, int D>
static hipError_t plan_t(const CompressArgs& a, hipStream_t s) {
  const size_t lds = stats_lds_bytes(B, a.nb_max);
  hipLaunchKernelGGL((k_stats<T, B, D>), dim3((unsigned)a.n_brow * a.H_s), dim3(B * 4), lds, s,
                     (const T*)a.Q, (const T*)a.K, a.H_s, a.T, a.info, a.order, a.n_brow, a.nb_max,
                     a.scale2, a.lse2, a.Mh);
  return hipGetLastError();
}

template <typename T, int B, int D>
static hipError_t gather_t(const CompressArgs& a, hipStream_t s) {
  const int HG = (a.H_s + 7) / 8;
  const uint64_t grid = (uint64_t)a.capacity * HG;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gather<T, B, D>), dim3((unsigned)grid), dim3(B * 4), 0, s, (const T*)a.Q,
                     (const T*)a.K, a.H_s, a.T, a.info, a.block_idx, a.block_row, a.counters,
                     a.capacity, a.lse2, a.scale2, a.probs, a.part);
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

static hipError_t stats_dispatch(const CompressArgs& a, hipStream_t s) { MF_DISPATCH_QK(plan_t, a, s); }
static hipError_t gather_dispatch(const CompressArgs& a, hipStream_t s) { MF_DISPATCH_QK(gather_t, a, s); }

hipError_t compress_plan(const CompressArgs& a, hipStream_t s) {
  hipError_t e = stats_dispatch(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_head_reduce, dim3(a.n_brow), dim3(256), 0, s, a.Mh, a.H_s, a.n_brow,
                     a.nb_max, a.info, a.M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int N = 1;
  while (N < a.nb_max) N <<= 1;
  const size_t lds = (size_t)N * (sizeof(double) + sizeof(int));
  hipLaunchKernelGGL(k_select, dim3(a.n_brow), dim3(256), lds, s, a.M, a.info, a.nb_max, a.H_s,
                     a.B, a.tau, a.flags, a.counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, a.counts, a.n_brow, a.capacity,
                     a.block_ptr, a.counters);
  return hipGetLastError();
}

hipError_t compress_fill(const CompressArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_emit, dim3(a.n_brow), dim3(256), 0, s, a.flags, a.block_ptr, a.info,
                     a.nb_max, a.capacity, a.block_idx, a.block_row);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = gather_dispatch(a, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowmass, dim3(a.n_brow, a.H_s), dim3(a.B), 0, s, a.part, a.block_ptr,
                     a.info, a.counters, a.H_s, a.B, a.T, a.capacity, a.rkm);
  return hipGetLastError();
}

}  // namespace mf
