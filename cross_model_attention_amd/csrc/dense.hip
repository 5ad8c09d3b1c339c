// Dense causal attention for the receiver layers that are recomputed, and the HBM copy probe.
//
// [Reuses Attention, attention-map section] (roboind.com): the receiver first computes a few
// layers normally to build its own hidden state; [Abstract]: partial recomputation.  These
// layers use plain causal softmax attention.
//
// k_attn runs the score sweep of the compression (sweep.h) with its attention half only: one
// workgroup per (pair of consecutive block rows of a sequence, query head), each key tile staged
// in LDS once for both rows; scores transposed (keys x queries) on MFMA, online softmax in base 2
// with the block maximum and block sum of exponentials, P.V on the fp16 MFMA from the prepared V
// tiles (V of the query head's KV head).
#include "sweep.h"

namespace mf {

// Work item: with a multiple of 8 query heads, the query heads (in KV-head order) are dealt to
// the XCDs in runs (workgroup b runs on XCD b mod 8), so the heads sharing one KV head, and the
// workgroups in flight on one XCD, read the same keys and values through one L2.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attn(const T* __restrict__ Q, const T* __restrict__ K,
                                              int H_q, int H_kv, int64_t T_tot,
                                              const int32_t* __restrict__ info,
                                              const int32_t* __restrict__ pairs, int n_pair, int n_brow,
                                              const uint16_t* __restrict__ vfrag,
                                              const int32_t* __restrict__ vexps, HeadMap hm, float scale2,
                                              float* __restrict__ O) {
  int hi, pr;
  if ((H_q & 7) == 0) {
    const int q = blockIdx.x >> 3;
    hi = (blockIdx.x & 7) * (H_q >> 3) + q / n_pair;
    pr = q % n_pair;
  } else {
    hi = blockIdx.x / n_pair;
    pr = blockIdx.x % n_pair;
  }
  const int g = hm.perm[hi], kv = hm.kv[g];
  const SweepHead<T> hd{Q + (size_t)g * D, (int64_t)H_q * D, K + (size_t)kv * D, (int64_t)H_kv * D, kv,
                        O + (size_t)g * D, (int64_t)H_q * D};
  sweep_body<T, 64, D, true, false>(hd, g, pr, T_tot, info, pairs, nullptr, 0, n_brow, 0, scale2, nullptr,
                                    nullptr, nullptr, AttnOut{vfrag, vexps});
}

bool dense_supported(int dtype, int d) {
  return (dtype == DT_F32 || dtype == DT_BF16) && (d == 64 || d == 128);
}

template <typename T, int D>
static hipError_t dense_t(const DenseArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<T, D>), dim3((unsigned)a.n_pair * a.H_q), dim3(256), 0, s, (const T*)a.Q,
                     (const T*)a.K, a.H_q, a.H_kv, a.T, a.info, a.pairs, a.n_pair, a.n_brow, a.vfrag, a.vexps,
                     a.hm, kLog2e / sqrtf((float)a.d), a.O);
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

// ------------------------------------------------------------------------------------------
// HBM read probe: grid-stride non-temporal 16-byte loads, 8 in flight per thread, folded by XOR;
// the fold is stored only when it equals one fixed 128-bit value, so the loads cannot be dropped.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_read(const v4u* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  v4u acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n; i += 8 * stride) {
    v4u x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0xF39CC060u && acc[3] == 0x5CEDC834u)
    sink[0] = acc[0] ^ acc[3];
}

// ------------------------------------------------------------------------------------------
// HBM write probe: coalesced non-temporal 16-byte stores (each wave instruction writes 1 KiB of
// contiguous memory).  Per iteration a workgroup writes 256 * 5 records; with a source it first
// reads 256 records (non-temporal) and the five records it writes from each are that record plus
// u = 0..4 in every 32-bit word, so no load can be dropped.  Without a source, record it * 1280 +
// 256 u + t holds {it, 7, 8, 9} + u.
// ------------------------------------------------------------------------------------------
template <bool RD>
__global__ __launch_bounds__(256) void k_write(v4u* __restrict__ dst, const v4u* __restrict__ src, size_t n_iter) {
  for (size_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
    v4u x = {(uint32_t)it, 7u, 8u, 9u};
    if (RD) x = __builtin_nontemporal_load(src + it * 256 + threadIdx.x);
    v4u* d = dst + it * 1280 + threadIdx.x;
#pragma unroll
    for (int u = 0; u < 5; ++u) __builtin_nontemporal_store(x + (uint32_t)u, d + u * 256);
  }
}

hipError_t write_probe(void* dst, size_t bytes, const void* src, hipStream_t s) {
  const size_t n_iter = bytes / (1280 * 16);
  if (n_iter == 0) return hipSuccess;
  const unsigned grid = 256 * 16;
  if (src)
    hipLaunchKernelGGL(k_write<true>, dim3(grid), dim3(256), 0, s, (v4u*)dst, (const v4u*)src, n_iter);
  else
    hipLaunchKernelGGL(k_write<false>, dim3(grid), dim3(256), 0, s, (v4u*)dst, nullptr, n_iter);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// HBM fill probe: plain (temporal) 16-byte stores of one 32-bit value, each workgroup iteration
// writing 256 KiB of contiguous memory (64 stores per thread; every wave instruction covers 1 KiB).
// Long contiguous runs and ordinary stores give the chip's write ceiling, which non-temporal
// stores in short runs do not reach.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fill(v4u* __restrict__ dst, size_t n_iter, uint32_t v) {
  const v4u x = {v, v, v, v};
  for (size_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
    v4u* d = dst + it * 16384 + threadIdx.x;
#pragma unroll 16
    for (int u = 0; u < 64; ++u) d[u * 256] = x;
  }
}

hipError_t fill_probe(void* dst, size_t bytes, uint32_t v, hipStream_t s) {
  const size_t n_iter = bytes / 262144;
  if (n_iter == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill, dim3(2048), dim3(256), 0, s, (v4u*)dst, n_iter, v);
  return hipGetLastError();
}

hipError_t read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned grid = 256 * 64;
  hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, s, (const v4u*)src, n, sink);
  return hipGetLastError();
}

}  // namespace mf
