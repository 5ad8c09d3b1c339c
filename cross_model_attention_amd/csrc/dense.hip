// Dense causal attention for the receiver layers that are recomputed, and the HBM copy probe.
//
// [Reuses Attention, attention-map section] (roboind.com): the receiver first computes a few
// layers normally to build its own hidden state; [Abstract]: partial recomputation.  These
// layers use plain causal softmax attention.
//
// k_dense: one workgroup (4 waves) per (64-query block row, query head); wave w owns queries
// 16w..16w+15.  Key tiles go through LDS once per workgroup; scores are formed transposed (keys x
// queries, MFMA bf16 or f32) so that each lane's probabilities for 2 x 4 keys are exactly one fp16
// MFMA operand slice in the key order of the prepared V tiles; P.V then runs on MFMA fp16 with V
// from those tiles.  Online softmax in base 2; the row maximum is shared by the four lane groups
// of a query column through the gfx950 row-swap permutes.
#include "common.h"
#include "kernels.h"

namespace mf {

template <typename T, int D>
struct DFrag;
template <int D>
struct DFrag<uint16_t, D> {
  static constexpr int N = D / 32;
  v8s v[N];
  __device__ __forceinline__ void load(const uint16_t* row, bool valid, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = valid ? as_v8s(ld16(row + 32 * k + 8 * a)) : as_v8s(zero_u4());
  }
  __device__ __forceinline__ void load_lds(const unsigned char* row, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = as_v8s(*reinterpret_cast<const v4u*>(row + (32 * k + 8 * a) * 2));
  }
  __device__ __forceinline__ v4f dot(const DFrag& o, v4f acc) const {
#pragma unroll
    for (int k = 0; k < N; ++k) acc = mfma_bf16(v[k], o.v[k], acc);
    return acc;
  }
};
template <int D>
struct DFrag<float, D> {
  static constexpr int N = D / 4;
  float v[N];
  __device__ __forceinline__ void load(const float* row, bool valid, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = valid ? row[4 * k + a] : 0.f;
  }
  __device__ __forceinline__ void load_lds(const unsigned char* row, int a) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = *reinterpret_cast<const float*>(row + (4 * k + a) * 4);
  }
  __device__ __forceinline__ v4f dot(const DFrag& o, v4f acc) const {
#pragma unroll
    for (int k = 0; k < N; ++k) acc = mfma_f32(v[k], o.v[k], acc);
    return acc;
  }
};

// Causal / padding mask of one key block, applied in place to the raw scores: keys after the
// query (and every key of a padding query) become -inf.  kq = the lane's first key minus its
// query.  Only the diagonal block and blocks of a partial row call it.
__device__ __forceinline__ void dense_mask(v4f (&s)[4], int kq, bool qvalid) {
  asm volatile("" : "+v"(kq));                     // keep the compares inside the block
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!(qvalid && kq + 16 * mt + i <= 0)) s[mt][i] = -__builtin_inff();
}

// One key block of the online softmax for this lane's query column: scores s[mt] (keys 16 mt +
// 4 a + i), running max m / sum l, output accumulators rescaled, then P.V with the prepared V
// tiles.
template <int D>
__device__ __forceinline__ void dense_block(v4f (&s)[4], float scale2, float& m, float& l,
                                            v4f (&acc)[D / 16], const uint16_t* vb) {
  constexpr int MT = 4, NCH = 2, NDT = D / 16;
  constexpr float kNegInf = -__builtin_inff();
  float tmax = kNegInf;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = s[mt][i] * scale2;
      s[mt][i] = x;
      tmax = __builtin_fmaxf(tmax, x);
    }
  tmax = xrow_max(tmax);
  const float mn = __builtin_fmaxf(m, tmax);
  // a column with nothing visible yet (padding rows) keeps a finite reference so every
  // exponential below is exactly 0; no lane-dependent branch around the MFMAs
  const float mref = mn == kNegInf ? 0.f : mn;
  const float alpha = fast_exp2(m - mref);
  l *= alpha;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[dt][i] *= alpha;
  m = mn;
  v8h pop[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    f2 pr[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = fast_exp2(s[2 * ch + (e >> 2)][e & 3] - mref);
      const float p1 = fast_exp2(s[2 * ch + ((e + 1) >> 2)][(e + 1) & 3] - mref);
      l += p0 + p1;
      pr[e / 2] = f2{p0 * 32768.f, p1 * 32768.f};
    }
    uint32_t pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pk[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr[q], h2));
    pop[ch] = as_v8h(v4u{pk[0], pk[1], pk[2], pk[3]});
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      acc[dt] = mfma_f16(as_v8h(ld16(vb + (ch * NDT + dt) * 512)), pop[ch], acc[dt]);
}

// k_dense: one workgroup (4 waves) per (64-query block row, query head); wave w owns queries
// 16w..16w+15.  Key tiles are loaded once per workgroup with coalesced 16-byte loads, two blocks
// ahead, and staged in LDS (row stride 32 mod 128 bytes: conflict-free operand reads); scores are
// formed transposed (keys x queries) on MFMA so each lane's probabilities for 2 x 4 keys are one
// fp16 MFMA operand slice in the key order of the prepared V tiles, read straight from memory.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_dense(const T* __restrict__ Q, const T* __restrict__ K,
                                               int H_q, int H_kv, int64_t T_tot,
                                               const int32_t* __restrict__ info,
                                               const int32_t* __restrict__ order, int n_brow,
                                               const uint16_t* __restrict__ vfrag,
                                               const int32_t* __restrict__ vexps, HeadMap hm,
                                               float scale2, float* __restrict__ O) {
  constexpr int B = 64, MT = 4, NCH = 2, NDT = D / 16;
  constexpr int NTHR = 256;
  constexpr int ROWB = D * (int)sizeof(T) + 32;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int CPT = B * CPR / NTHR;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2][B * ROWB];
  const int g = blockIdx.x % H_q;
  const int brow = order[blockIdx.x / H_q];
  const BrowInfo bi = load_info(info, brow);
  const int kv = hm.kv[g];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, a = lane >> 4, c = lane & 15;
  const int rows = min(B, bi.n - bi.I * B);
  const int qrow = 16 * w + c;                       // query of this lane's column
  const int qloc = bi.I * B + qrow;
  const bool qvalid = qrow < rows;

  DFrag<T, D> qf;
  qf.load(Q + ((size_t)(bi.tok0 + qrow) * H_q + g) * D, qvalid, a);
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K + ((size_t)bi.seq0 * H_kv + kv) * D);
  const size_t kstride = (size_t)H_kv * D * sizeof(T);
  const int kbrow0 = brow - bi.I;

  auto fetch_k = [&](v4u (&kst)[CPT], int J) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int piece = threadIdx.x + u * NTHR;
      const int row = piece / CPR, col = piece % CPR;
      const int key = J * B + row;
      kst[u] = key < bi.n ? ld16(Kb + (size_t)key * kstride + col * 16) : zero_u4();
    }
  };
  auto stage_k = [&](const v4u (&kst)[CPT], int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int piece = threadIdx.x + u * NTHR;
      *reinterpret_cast<v4u*>(&s_k[buf][(piece / CPR) * ROWB + (piece % CPR) * 16]) = kst[u];
    }
  };

  float m = -__builtin_inff(), l = 0.f;
  v4f acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero4();
  const bool partial = rows < B;

  auto block = [&](int J, v4u (&fill)[CPT], const v4u (&next)[CPT]) {
    if (J + 2 <= bi.I) fetch_k(fill, J + 2);
    const unsigned char* kt = s_k[J & 1];
    v4f s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      DFrag<T, D> kf;
      kf.load_lds(kt + (16 * mt + c) * ROWB, a);
      s[mt] = kf.dot(qf, zero4());
    }
    const uint16_t* vb = vfrag + ((((size_t)kv * n_brow + kbrow0 + J) * NCH) * NDT) * 512 + lane * 8;
    if (J == bi.I || partial) dense_mask(s, J * B + 4 * a - qloc, qvalid);
    dense_block<D>(s, scale2, m, l, acc, vb);
    if (J + 1 <= bi.I) stage_k(next, (J + 1) & 1);
    __syncthreads();
  };
  v4u k0[CPT], k1[CPT];
  fetch_k(k0, 0);
  if (bi.I >= 1) fetch_k(k1, 1);
  stage_k(k0, 0);
  __syncthreads();
  for (int J = 0; J <= bi.I; J += 2) {
    block(J, k0, k1);
    if (J + 1 <= bi.I) block(J + 1, k1, k0);
  }
  l = xrow_sum(l);
  if (!qvalid) return;
  const float inv = ldexpf(1.f, -15 - vexps[kv]) / l;
  float* orow = O + ((size_t)(bi.tok0 + qrow) * H_q + g) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * a + i] = acc[dt][i] * inv;
}

bool dense_supported(int dtype, int d) {
  return (dtype == DT_F32 || dtype == DT_BF16) && (d == 64 || d == 128);
}

template <typename T, int D>
static hipError_t dense_t(const DenseArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_dense<T, D>), dim3((unsigned)a.n_brow * a.H_q), dim3(256), 0, s,
                     (const T*)a.Q, (const T*)a.K, a.H_q, a.H_kv, a.T, a.info, a.order, a.n_brow,
                     a.vfrag, a.vexps, a.hm, kLog2e / sqrtf((float)a.d), a.O);
  return hipGetLastError();
}

hipError_t dense_attention(const DenseArgs& a, hipStream_t s) {
  if (a.dtype == DT_BF16) return a.d == 128 ? dense_t<uint16_t, 128>(a, s) : dense_t<uint16_t, 64>(a, s);
  return a.d == 128 ? dense_t<float, 128>(a, s) : dense_t<float, 64>(a, s);
}

// ------------------------------------------------------------------------------------------
// HBM copy probe: grid-stride 16-byte copy, 4 loads in flight per thread.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_copy(v4u* __restrict__ dst, const v4u* __restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(x0, dst + i);
    __builtin_nontemporal_store(x1, dst + i + stride);
    __builtin_nontemporal_store(x2, dst + i + 2 * stride);
    __builtin_nontemporal_store(x3, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t copy_probe(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned grid = 256 * 16;
  hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, s, (v4u*)dst, (const v4u*)src, n);
  return hipGetLastError();
}

}  // namespace mf
