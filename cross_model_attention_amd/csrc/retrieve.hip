// Fused retrieve: kept sender blocks -> receiver attention output, plus the V preparation it
// reads.
//
// [MapFlow开源, section 算得省的:融合内核执行] (aitest123.com) and [Reuses Attention, third
// component] (roboind.com): the kernel reads the sparse blocks, performs the linear combination
// of sender heads into receiver heads in on-chip memory, multiplies by the receiver's own V and
// accumulates, writing only the output.  Neither the dense map nor the mixed map touches HBM.
//
// k_retrieve, one workgroup (8 waves) per (block row, 16-row tile, head split); a split holds up
// to 24 receiver heads, or 32 on the half-block path (each block taken as two 32-key halves):
//   for each kept block J of the row, in column order:
//     stage 1  head mix on MFMA (bf16): Ahat[g, i, j] = sum_h Ws[g, h] P[h, i, j] for the 16 rows
//              x B keys, where Ws = W * 2^s_g is split into bf16 hi + lo parts so the product
//              with the exactly-bf16 P keeps ~16 bits of W; the fp32 sums are rounded to fp16
//              and staged in LDS (double buffered)
//     stage 2  P.V on MFMA (fp16): O[g] += Ahat[g] V[kv(g)] with V from the prepared fp16
//              operand tiles (L2-resident: each V block is shared by every row that keeps it)
//   epilogue   O = acc * 2^-t_kv / den, den[g, i] = sum_h Ws[g, h] row_kept_mass[h, i] (den and
//              acc both carry 2^s_g)
// The kept-block probabilities are streamed once with non-temporal loads; the next block's tile
// is fetched into registers while the current block's P.V runs.
#include "common.h"
#include "kernels.h"

namespace mf {

// ------------------------------------------------------------------------------------------
// V preparation
// ------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load_v(const T* V, int64_t idx);
template <>
__device__ __forceinline__ float load_v<uint16_t>(const uint16_t* V, int64_t idx) {
  return bf16_to_f32(V[idx]);
}
template <>
__device__ __forceinline__ float load_v<float>(const float* V, int64_t idx) {
  return V[idx];
}

// element offset of (token-in-sequence kloc, kv head, column d) for contiguous or paged V
__device__ __forceinline__ int64_t v_offset(const BrowInfo& bi, int seq, int kloc, int kv, int d,
                                            int H_kv, int D, const int32_t* page_table,
                                            int page_size, int pages_per_seq) {
  if (page_table == nullptr) return ((int64_t)(bi.seq0 + kloc) * H_kv + kv) * D + d;
  const int page = page_table[(int64_t)seq * pages_per_seq + kloc / page_size];
  return (((int64_t)page * page_size + kloc % page_size) * H_kv + kv) * D + d;
}

__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// One workgroup per (group of block rows, KV head): block rows brow = blockIdx.x + k gridDim.x.
template <typename T>
__global__ __launch_bounds__(256) void k_vmax(const T* __restrict__ V, int H_kv, int D, int B, int n_brow,
                                              const int32_t* __restrict__ info,
                                              const int32_t* __restrict__ brow_seq,
                                              const int32_t* __restrict__ page_table,
                                              int page_size, int pages_per_seq,
                                              uint32_t* __restrict__ vmax_bits) {
  __shared__ float red[4];
  const int kv = blockIdx.y;
  // 16-byte loads: a token's D values of one KV head are contiguous in either layout
  constexpr int EPC = 16 / (int)sizeof(T);         // elements per 16-byte chunk
  const int CH = D / EPC;                          // chunks per token row
  float m = 0.f;
  for (int brow = blockIdx.x; brow < n_brow; brow += gridDim.x) {
  const BrowInfo bi = load_info(info, brow);
  const int seq = brow_seq[brow];
  for (int e = threadIdx.x; e < B * CH; e += blockDim.x) {
    const int kloc = bi.I * B + e / CH;
    if (kloc < bi.n) {
      const v4u x = ld16(V + v_offset(bi, seq, kloc, kv, (e % CH) * EPC, H_kv, D, page_table, page_size,
                                      pages_per_seq));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2) {
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(x[j] & 0xFFFFu))));
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(x[j] >> 16))));
        } else {
          m = fmaxf(m, fabsf(__uint_as_float(x[j])));
        }
      }
    }
  }
  }
  // NaN must win the maximum so that the scale falls back to 1
  if (m != m) m = __uint_as_float(0x7FC00000u);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int r = 1; r < (int)(blockDim.x >> 6); ++r) t = fmaxf(t, red[r]);
    atomicMax(&vmax_bits[kv], __float_as_uint(t));
  }
}

__global__ void k_vexps(const uint32_t* __restrict__ vmax_bits, int H_kv, int32_t* __restrict__ exps) {
  const int kv = threadIdx.x;
  if (kv >= H_kv) return;
  const float m = __uint_as_float(vmax_bits[kv]);
  int e = 0;
  if (m > 0.f && m < __builtin_inff()) {
    int ex;
    frexpf(m, &ex);          // m <= 2^ex
    e = 15 - ex;
    e = max(-100, min(100, e));
  }
  exps[kv] = e;
}

// One workgroup per (block row, KV head).  The block's V rows are staged in LDS with 16-byte
// loads (zero past the sequence's end), then each thread writes 16-byte operand records: lane
// (a, dd) of tile (kv, block row, 32-key chunk, 16-column slice) holds V[key(e)][kv][16 dt + dd]
// for e = 0..7, where within the chunk key(e) = 4a + e for e < 4 and 16 + 4a + (e - 4) otherwise.
// That key order matches the accumulator layout of two stacked 16x16 score tiles, so attention
// probabilities computed in registers can be used as the other MFMA operand without a
// transpose.  The records of one (KV head, block row) are contiguous.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_vconvert(const T* __restrict__ V, int H_kv, int B,
                                                  int n_brow, const int32_t* __restrict__ info,
                                                  const int32_t* __restrict__ brow_seq,
                                                  const int32_t* __restrict__ page_table,
                                                  int page_size, int pages_per_seq,
                                                  const int32_t* __restrict__ exps,
                                                  uint16_t* __restrict__ frag) {
  constexpr int NDT = D / 16;
  constexpr int ROW = D * (int)sizeof(T) + 16;    // staged row stride: keys 4 a + e fall on distinct banks
  constexpr int CH = D * (int)sizeof(T) / 16;     // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) unsigned char s_v[64 * ROW];
  const int brow = blockIdx.x, kv = blockIdx.y;
  const BrowInfo bi = load_info(info, brow);
  const int seq = brow_seq[brow];
  for (int e = threadIdx.x; e < B * CH; e += blockDim.x) {
    const int key = e / CH, chunk = e % CH;
    const int kloc = bi.I * B + key;
    v4u x = zero_u4();
    if (kloc < bi.n)
      x = ld16(V + v_offset(bi, seq, kloc, kv, chunk * (16 / (int)sizeof(T)), H_kv, D, page_table, page_size,
                            pages_per_seq));
    *reinterpret_cast<v4u*>(s_v + key * ROW + chunk * 16) = x;
  }
  __syncthreads();
  const float scale = ldexpf(1.f, exps[kv]);
  const int NCH = B / 32;
  const int n_rec = NCH * NDT * 64;
  uint16_t* out = frag + ((size_t)kv * n_brow + brow) * (size_t)n_rec * 8;
  for (int r = threadIdx.x; r < n_rec; r += blockDim.x) {
    const int lane = r & 63, dt = (r >> 6) % NDT, ch = (r >> 6) / NDT;
    const int a = lane >> 4, dd = lane & 15;
    const int col = 16 * dt + dd;
    uint32_t packed[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t two = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * p + q;
        const int koff = 32 * ch + (e < 4 ? 4 * a + e : 16 + 4 * a + (e - 4));
        float v;
        if constexpr (sizeof(T) == 2) v = bf16_to_f32(*reinterpret_cast<const uint16_t*>(s_v + koff * ROW + col * 2));
        else v = *reinterpret_cast<const float*>(s_v + koff * ROW + col * 4);
        two |= (uint32_t)f32_to_f16_bits(v * scale) << (16 * q);
      }
      packed[p] = two;
    }
    st16(out + (size_t)r * 8, v4u{packed[0], packed[1], packed[2], packed[3]});
  }
}

template <typename T, int D>
static hipError_t vconvert_t(const VprepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_vconvert<T, D>), dim3(a.n_brow, a.H_kv), dim3(256), 0, s, (const T*)a.V, a.H_kv, a.B,
                     a.n_brow, a.info, a.brow_seq, a.page_table, a.page_size, a.pages_per_seq,
                     a.exps, a.frag);
  return hipGetLastError();
}

hipError_t v_prepare(const VprepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, s, a.vmax_bits, a.H_kv, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_brow < 1) {                              // no tokens: scale exponents only
    hipLaunchKernelGGL(k_vexps, dim3(1), dim3(64), 0, s, a.vmax_bits, a.H_kv, a.exps);
    return hipGetLastError();
  }
  if (a.dtype == DT_BF16)
    hipLaunchKernelGGL((k_vmax<uint16_t>), dim3(min(a.n_brow, 64), a.H_kv), dim3(256), 0, s,
                       (const uint16_t*)a.V, a.H_kv, a.d, a.B, a.n_brow, a.info, a.brow_seq, a.page_table,
                       a.page_size, a.pages_per_seq, a.vmax_bits);
  else
    hipLaunchKernelGGL((k_vmax<float>), dim3(min(a.n_brow, 64), a.H_kv), dim3(256), 0, s,
                       (const float*)a.V, a.H_kv, a.d, a.B, a.n_brow, a.info, a.brow_seq, a.page_table,
                       a.page_size, a.pages_per_seq, a.vmax_bits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_vexps, dim3(1), dim3(64), 0, s, a.vmax_bits, a.H_kv, a.exps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dtype == DT_BF16) return a.d == 128 ? vconvert_t<uint16_t, 128>(a, s) : vconvert_t<uint16_t, 64>(a, s);
  return a.d == 128 ? vconvert_t<float, 128>(a, s) : vconvert_t<float, 64>(a, s);
}

// ------------------------------------------------------------------------------------------
// k_retrieve
// ------------------------------------------------------------------------------------------
constexpr int RT_ROWS = 16;     // rows per work item
constexpr int RT_WAVES = 8;     // waves per workgroup
constexpr int ROWS_PER_WAVE = RT_ROWS / RT_WAVES;

// LDS layout of the mixed map: [head][row][key] fp16, 160-byte rows and 2592-byte heads (16 rows
// plus 32 bytes), two buffers of up to 24 heads.  The 16-byte stage-2 reads (lane (a, c): row c,
// key chunk a) and stage-1 writes (lane (a, c): head c, key chunk a) see strides of 32 mod 128
// bytes; the LDS conflict counters read about 0.9 conflict cycles per LDS-active cycle with them
// and half that with strides of 16 mod 128, at the same kernel time.
template <int B, int HP, bool HALF = false>
struct AhatLayout {
  static_assert(HP <= 3 && B * 2 <= 160, "whole-block buffers hold up to 24 heads of up to 80 keys");
  static constexpr int kRowBytes = 160;
  static constexpr int kHeadBytes = RT_ROWS * kRowBytes + 32;
};
// HALF: the mixed map of one 32-key half block at a time, 80-byte rows, 1296-byte heads
template <int B, int HP>
struct AhatLayout<B, HP, true> {
  static constexpr int kRowBytes = 80;
  static constexpr int kHeadBytes = RT_ROWS * kRowBytes + 16;
};

// Per-slot receiver data of a work item: the slot's weight row, its V operand tiles (KV head
// already applied), its output column block and row stride, and V's scale exponent.
struct SlotInfo {
  const MF_GLOBAL float* w;
  const MF_GLOBAL uint16_t* v;
  MF_GLOBAL float* o;
  MF_GLOBAL float* dn;   // running denominator of the head (cross-layer accumulation), row stride H_r
  int ostride;
  int vexp;
};

// Head mix on MFMA: N-tiles are the split's receiver heads in chunks of 16 (NTG = ceil(HP / 2)
// tiles), the contraction runs over the sender heads twice, once against the bf16 "hi" part and
// once against the bf16 "lo" part of the scaled weights, accumulating into the same fp32 tile:
// Ws = hi + lo keeps ~16 bits of W while the kept probabilities enter the MFMA exactly.  A split
// holds up to 8*HP heads; each of the 8 waves owns HP of them in stage 2.
//
// Work items are XCD-aware: the row tiles and head splits of one block row share an XCD and run
// one after the other, so every split after the first finds the P tile in that XCD's L2.  A
// split's slots may hold heads of different receivers (a fan-out): each slot carries its own
// weights, V and output.
template <int B, int D, int HP, int KC, bool FAST, bool HALF = false>
__global__ __launch_bounds__(RT_WAVES * 64) void k_retrieve(const RetrieveArgs args) {
  const uint16_t* __restrict__ probs = args.probs;
  const int32_t* __restrict__ block_ptr = args.block_ptr;
  const int32_t* __restrict__ block_idx = args.block_idx;
  const int32_t* __restrict__ info = args.info;
  const int32_t* __restrict__ order = args.order;
  const int64_t capacity = args.capacity;
  const int n_brow = args.n_brow, H_s = args.H_s;
  const int64_t T_tot = args.T;
  const float* __restrict__ rkm = args.rkm;
  constexpr int MT = B / 16;               // 16-key M-tiles per row
  constexpr int NCH = B / 32;              // 32-key chunks per block
  constexpr int NDT = D / 16;              // 16-column output tiles
  constexpr int RB = AhatLayout<B, HP, HALF>::kRowBytes;
  constexpr int GB = AhatLayout<B, HP, HALF>::kHeadBytes;
  static_assert(!HALF || (FAST && B == 64), "the half-block schedule is a fast path for B = 64");
  constexpr int HR_MAX = 8 * HP;
  constexpr int NTG = (HP + 1) / 2;        // 16-head N-tiles of the mix
  constexpr int HPW = HP;                  // stage 2: wave w owns slots w HP .. w HP + HP - 1

  __shared__ __attribute__((aligned(16))) unsigned char s_ahat[2][HR_MAX * GB];
  __shared__ float s_den[HR_MAX][RT_ROWS];
  __shared__ int s_sexp[HR_MAX];
  __shared__ int s_head[HR_MAX];
  __shared__ SlotInfo s_slot[HR_MAX];
  __shared__ v4u s_wop[NTG][KC][2][64];

  constexpr int NRT = B / RT_ROWS;         // row tiles per block row
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int q = b >> 3;
  const int rt = q % NRT;
  const int n_split = args.n_split;
  const int split = (q / NRT) % n_split;
  const int gidx = (q / (NRT * n_split)) * 8 + xcd;
  if (gidx >= args.n_order) return;
  const int brow = order[gidx];
  const BrowInfo bi = load_info(info, brow);
  const int rows_blk = min(B, bi.n - bi.I * B);
  const int rows = min(RT_ROWS, rows_blk - RT_ROWS * rt);
  if (rows <= 0) return;
  const int row0 = RT_ROWS * rt;              // first row of the tile within the block row
  const int HGp = (H_s + 7) >> 3;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, a = lane >> 4, c = lane & 15;
  // this workgroup's heads: slot j (j = 0..HR_MAX-1) holds head slot_head[split][j] (-1: empty;
  // heads fill the leading slots) of receiver slot_recv[split][j], KV head slot_kv[split][j];
  // mixed maps, weights and denominators are indexed by the slot
  const int n_slots = args.split_nslots[split];
  if (threadIdx.x < HR_MAX) {
    const int j = threadIdx.x;
    const int g = args.slot_head[split][j];
    s_head[j] = g;
    // an empty slot still names valid V tiles (receiver 0, KV head 0): a wave whose first slot
    // is empty prefetches them and never uses them
    const RecvArgs& rv = args.recv[args.slot_recv[split][j]];
    const int kv = args.slot_kv[split][j];
    SlotInfo si{nullptr, (const MF_GLOBAL uint16_t*)(rv.vfrag + (size_t)kv * n_brow * (NCH * NDT * 512)),
                nullptr, nullptr, 0, 0};
    if (g >= 0) {
      si.w = (const MF_GLOBAL float*)(rv.W + (size_t)g * H_s);
      si.o = (MF_GLOBAL float*)(rv.O + (size_t)g * D);
      si.dn = rv.den ? (MF_GLOBAL float*)(rv.den + g) : nullptr;
      si.ostride = rv.H_r * D;
      si.vexp = rv.vexps[kv];
    }
    s_slot[j] = si;
  }
  __syncthreads();
  auto head_of = [&](int j) { return s_head[j]; };

  // ---- setup: per-head scale, scaled weights, denominators ---------------------------------
  // The raw weights of every slot and the kept row masses of the tile's rows are read with one
  // coalesced pass each into the second mixed-map buffer (unused until the loop); everything
  // else is computed from LDS.  Read element by element, these would be dozens of dependent
  // global round trips per workgroup.
  float (*s_x)[64] = reinterpret_cast<float (*)[64]>(s_ahat[1]);
  float (*s_rk)[RT_ROWS] = reinterpret_cast<float (*)[RT_ROWS]>(s_ahat[1] + HR_MAX * 64 * sizeof(float));
  static_assert(HR_MAX * 64 * sizeof(float) + 64 * RT_ROWS * sizeof(float) <= HR_MAX * GB,
                "weights and kept masses fit in one Ahat buffer");
  for (int t = threadIdx.x; t < HR_MAX * 64; t += blockDim.x) {
    const int j = t >> 6, h = t & 63;
    s_x[j][h] = (head_of(j) >= 0 && h < H_s) ? s_slot[j].w[h] : 0.f;
  }
  for (int t = threadIdx.x; t < H_s * RT_ROWS; t += blockDim.x) {
    const int h = t / RT_ROWS, i = t % RT_ROWS;
    s_rk[h][i] = i < rows ? rkm[(size_t)h * T_tot + bi.tok0 + row0 + i] : 0.f;
  }
  __syncthreads();
  // per-slot scale: 2^s with sum_h |W| 2^s <= 2^15
  if (threadIdx.x < HR_MAX) {
    int e = 0;
    if (head_of(threadIdx.x) >= 0) {
      float sa = 0.f;
#pragma unroll 8
      for (int h = 0; h < H_s; ++h) sa += fabsf(s_x[threadIdx.x][h]);
      if (sa > 0.f && sa < __builtin_inff()) {
        int ex;
        frexpf(sa, &ex);      // sum |W| <= 2^ex
        e = max(-100, min(100, 15 - ex));
      }
    }
    s_sexp[threadIdx.x] = e;
  }
  __syncthreads();
  // scaled weights x = W 2^s (fp32), in place
  for (int t = threadIdx.x; t < HR_MAX * 64; t += blockDim.x) {
    const int j = t >> 6, h = t & 63;
    s_x[j][h] = ldexpf(s_x[j][h], s_sexp[j]);
  }
  __syncthreads();
  // denominators with the weights the mix uses: hi + lo, hi = bf16(x), lo = bf16(x - hi)
  for (int t = threadIdx.x; t < HR_MAX * RT_ROWS; t += blockDim.x) {
    const int j = t / RT_ROWS, i = t % RT_ROWS;
    float den = 0.f;
    // unrolled so that the LDS reads of several terms are in flight at once; the sum keeps its order
    if (head_of(j) >= 0 && i < rows)
#pragma unroll 8
      for (int h = 0; h < H_s; ++h) {
        const float x = s_x[j][h];
        const float hi = bf16_to_f32(f32_to_bf16(x));
        const float lo = bf16_to_f32(f32_to_bf16(x - hi));
        den += (hi + lo) * s_rk[h][i];
      }
    s_den[j][i] = den;
  }

  // stage-1 B operands (weights of virtual heads, bf16 hi / lo, head dims 32kc + 8a + e), kept in
  // LDS per lane and read on use: registers stay free for the operand prefetches
  if (w == 0) {
#pragma unroll
    for (int nt = 0; nt < NTG; ++nt) {
      const int jn = 16 * nt + c;
      const bool live = jn < HR_MAX && head_of(jn) >= 0;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int lo = 0; lo < 2; ++lo) {
          uint32_t pk[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t two = 0;
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const int h = 32 * kc + 8 * a + 2 * e2 + q2;
              uint32_t bits = 0;
              if (live && h < H_s) {
                const float x = s_x[jn][h];
                const uint16_t hb = f32_to_bf16(x);
                bits = lo ? f32_to_bf16(x - bf16_to_f32(hb)) : hb;
              }
              two |= bits << (16 * q2);
            }
            pk[e2] = two;
          }
          s_wop[nt][kc][lo][lane] = v4u{pk[0], pk[1], pk[2], pk[3]};
        }
    }
  }

  // stage-2 ownership: local slots s0 .. s0+HPW-1, all output tiles
  const int s0 = w * HPW;
  int sg[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) sg[j] = head_of(s0 + j);
  v4f acc[HPW][NDT];
#pragma unroll
  for (int j = 0; j < HPW; ++j)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[j][dt] = zero4();

  const int t0 = (int)min((int64_t)block_ptr[brow], capacity);
  const int t1 = (int)min((int64_t)block_ptr[brow + 1], capacity);
  const size_t blk_elems = (size_t)HGp * B * B * 8;
  const int kbrow0 = brow - bi.I;          // block row holding key block 0 of this sequence

  // P operands of this wave: rows ROWS_PER_WAVE*w + rr, all M-tiles, KC head chunks.  The loads
  // are unconditional: a head group past the last (when H_s is not a multiple of 32) reads the
  // last group again, whose products meet zero weights in the mix, and the prefetch past the
  // row's last block re-reads that block.  Conditional loads would make the compiler's wait
  // counts conservative, and vector-memory loads retire in order: a wait for a later load (a V
  // tile) would then also wait for the whole prefetch of the next block.
  // HALF holds the M-tiles of one 32-key half block (2h, 2h + 1), else all of the block's.
  constexpr int PM = HALF ? 2 : MT;
  v4u pa[ROWS_PER_WAVE][PM][KC];
  size_t p_off[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) p_off[kc] = (size_t)min(4 * kc + a, HGp - 1) * B * B * 8;
  auto load_p = [&](int t, int h = 0) {
    const uint16_t* pb = probs + (size_t)t * blk_elems;
#pragma unroll
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
      const int r = row0 + ROWS_PER_WAVE * w + rr;
#pragma unroll
      for (int mt = 0; mt < PM; ++mt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          pa[rr][mt][kc] = ld16_nt(pb + p_off[kc] + ((size_t)r * B + 16 * (mt + PM * h) + c) * 8);
    }
  };
  if (t0 < t1) load_p(t0);
  __syncthreads();

  // V operand tiles of the wave's first slot for key chunk 0 are fetched before the head mix,
  // so their latency hides under it; later chunks and other V heads are loaded on use.
  const MF_GLOBAL uint16_t* vj[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) vj[j] = s_slot[s0 + j].v + lane * 8;
  const MF_GLOBAL uint16_t* const v0 = vj[0];
  auto vtile = [&](const MF_GLOBAL uint16_t* vb, int kbrow, int ch) {
    return vb + (((size_t)kbrow * NCH + ch) * NDT) * 512;
  };
  // ---- stage 1: head mix -> fp16 Ahat in LDS (rows of this wave, every head of the split) ----
  // (HALF: the one 32-key chunk held in pa, into a half-block buffer)
  constexpr int NCM = HALF ? 1 : NCH;
  auto mix = [&](unsigned char* buf) {
#pragma unroll
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
      const int ii = ROWS_PER_WAVE * w + rr;
#pragma unroll
      for (int ch = 0; ch < NCM; ++ch) {
#pragma unroll
        for (int nt = 0; nt < NTG; ++nt) {
          v4f mx[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            v4f m4 = zero4();
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              const v8s p8 = as_v8s(pa[rr][2 * ch + half][kc]);
              m4 = mfma_bf16(p8, as_v8s(s_wop[nt][kc][0][lane]), m4);
              m4 = mfma_bf16(p8, as_v8s(s_wop[nt][kc][1][lane]), m4);
            }
            mx[half] = m4;
          }
          // lane (a, c): local head 16 nt + c, keys 32 ch + 16 half + 4a + i -> 8 fp16 values
          const int g = 16 * nt + c;
          if (g < n_slots) {                             // the slot holds a head
            uint32_t pk[4];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
              for (int p2 = 0; p2 < 2; ++p2) {
                const f2 v2 = {mx[half][2 * p2], mx[half][2 * p2 + 1]};
                pk[2 * half + p2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, h2));
              }
            *reinterpret_cast<v4u*>(buf + g * GB + ii * RB + (ch * 4 + a) * 16) = v4u{pk[0], pk[1], pk[2], pk[3]};
          }
        }
      }
      }
  };

  // FAST: every slot of every wave holds a head and a wave's heads share one V group (they belong
  // to one KV head of one receiver, as with grouped-query receivers; the host checks it).
  // Straight-line loads, software-pipelined in consumption order: a key chunk's V tiles for the
  // next block are requested right after this block's last product with them, and the next
  // block's P right after the mix.  In issue order every wait of a block then covers only older
  // loads (vector-memory loads retire in order), and each load has a whole stage to land.
  if constexpr (HALF) {
    // 32 heads: a block as two 32-key halves, each with its own mixed-map buffer and barrier, so
    // that only one half's P and V operands are held; the next half's are requested right after
    // the mix and the products of this one
    v8h vt[NDT];
    auto load_v = [&](int t, int h) {
      const MF_GLOBAL uint16_t* vb = vtile(v0, kbrow0 + block_idx[t], h);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vt[dt] = as_v8h(ld16(vb + dt * 512));
    };
    if (t0 < t1) load_v(t0, 0);
    for (int t = t0; t < t1; ++t) {
      const int tn = min(t + 1, t1 - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned char* buf = s_ahat[h];
        mix(buf);
        if (h == 0) load_p(t, 1);
        else load_p(tn, 0);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          const v8h aop = as_v8h(*reinterpret_cast<const v4u*>(buf + (s0 + j) * GB + c * RB + a * 16));
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[j][dt] = mfma_f16(aop, vt[dt], acc[j][dt]);
        }
        if (h == 0) load_v(t, 1);
        else load_v(tn, 0);
      }
    }
  } else if constexpr (FAST) {
    v8h vt[NCH][NDT];
    auto load_v = [&](int t, int ch) {
      const MF_GLOBAL uint16_t* vb = vtile(v0, kbrow0 + block_idx[t], ch);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vt[ch][dt] = as_v8h(ld16(vb + dt * 512));
    };
    if (t0 < t1) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) load_v(t0, ch);
    }
    for (int t = t0; t < t1; ++t) {
      unsigned char* buf = s_ahat[(t - t0) & 1];
      const int tn = min(t + 1, t1 - 1);
      mix(buf);
      load_p(tn);
      __syncthreads();
      // ---- stage 2: P.V for this wave's receiver heads ----
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          const v8h aop = as_v8h(*reinterpret_cast<const v4u*>(buf + (s0 + j) * GB + c * RB + (ch * 4 + a) * 16));
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[j][dt] = mfma_f16(aop, vt[ch][dt], acc[j][dt]);
        }
        load_v(tn, ch);
      }
    }
  } else {
  for (int t = t0; t < t1; ++t) {
    unsigned char* buf = s_ahat[(t - t0) & 1];
    const int J = block_idx[t];
    const int kbrow = kbrow0 + J;
    v8h vpre[NCH][NDT];
    {
      const MF_GLOBAL uint16_t* vb = vtile(v0, kbrow, 0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vpre[0][dt] = as_v8h(ld16(vb + dt * 512));
    }
    mix(buf);
    load_p(min(t + 1, t1 - 1));
    __syncthreads();
    // ---- stage 2: P.V for this wave's receiver heads and output tiles ----
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch > 0) {
        const MF_GLOBAL uint16_t* vb = vtile(v0, kbrow, ch);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vpre[ch][dt] = as_v8h(ld16(vb + dt * 512));
      }
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int g = sg[j];
        if (g < 0) continue;
        v8h vop[NDT];
        if (vj[j] == v0) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vop[dt] = vpre[ch][dt];
        } else {
          const MF_GLOBAL uint16_t* vb = vtile(vj[j], kbrow, ch);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vop[dt] = as_v8h(ld16(vb + dt * 512));
        }
        const v8h aop = as_v8h(*reinterpret_cast<const v4u*>(buf + (s0 + j) * GB + c * RB + (ch * 4 + a) * 16));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[j][dt] = mfma_f16(aop, vop[dt], acc[j][dt]);
      }
    }
  }
  }

  // ---- epilogue ----
  __syncthreads();
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int g = sg[j];
    if (g < 0) continue;
    // den carries the same 2^s_g as the mixed map, so only V's scale is undone here
    const SlotInfo& si = s_slot[s0 + j];
    const float unscale = ldexpf(1.f, -si.vexp);
    if (args.accumulate == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = 4 * a + i;
        if (ii >= rows) continue;
        const float inv = unscale / s_den[s0 + j][ii];
        MF_GLOBAL float* orow = si.o + (size_t)(bi.tok0 + row0 + ii) * si.ostride;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) orow[16 * dt + c] = acc[j][dt][i] * inv;
      }
    } else {
      // cross-layer mix: this layer's unnormalised output and denominator in true units (the
      // head's weight scale 2^s_g undone), summed over the layers, divided by the last one
      const float wun = ldexpf(1.f, -s_sexp[s0 + j]);
      const int mode = args.accumulate;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = 4 * a + i;
        if (ii >= rows) continue;
        const size_t tok = (size_t)(bi.tok0 + row0 + ii);
        MF_GLOBAL float* orow = si.o + tok * si.ostride;
        MF_GLOBAL float* dp = si.dn + tok * (si.ostride / D);
        float den = s_den[s0 + j][ii] * wun;
        if (mode >= 2) den += *dp;
        const float num = unscale * wun;
        const float inv = mode == 3 ? 1.f / den : 1.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          float v = acc[j][dt][i] * num;
          if (mode >= 2) v += orow[16 * dt + c];
          orow[16 * dt + c] = v * inv;
        }
        // modes 1 and 2 store the running denominator (lane column 0 of the slot's wave), mode 3
        // only reads it
        if (mode != 3 && c == 0) *dp = den;
      }
    }
  }
}

bool retrieve_supported(int B, int d, int H_r, int H_s) {
  return (B == 32 || B == 64) && (d == 64 || d == 128) && H_r >= 1 && H_r <= 48 && H_s >= 1 &&
         H_s <= 64;
}

template <int B, int D, int HP, int KC, bool FAST, bool HALF = false>
static hipError_t retrieve_t(const RetrieveArgs& a, hipStream_t s) {
  constexpr int NRT = B / RT_ROWS;
  const unsigned groups = (unsigned)((a.n_order + 7) / 8);
  hipLaunchKernelGGL((k_retrieve<B, D, HP, KC, FAST, HALF>), dim3(groups * 8 * NRT * a.n_split), dim3(RT_WAVES * 64), 0,
                     s, a);
  return hipGetLastError();
}

template <int B, int D>
static hipError_t retrieve_bd(const RetrieveArgs& a, hipStream_t s) {
  const int KC = ((a.H_s + 7) / 8 + 3) / 4;
  // 4 heads per wave: only the half-block fast path (B = 64)
  if (a.HP == 4) {
    if constexpr (B == 64) {
      if (a.fast && KC == 1) return retrieve_t<B, D, 4, 1, true, true>(a, s);
      if (a.fast && KC == 2) return retrieve_t<B, D, 4, 2, true, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
  // the fast path does not fit the register file with 3 heads per wave and two head chunks
  if (a.fast && !(a.HP == 3 && KC == 2)) {
    switch (a.HP * 4 + KC) {
      case 1 * 4 + 1: return retrieve_t<B, D, 1, 1, true>(a, s);
      case 2 * 4 + 1: return retrieve_t<B, D, 2, 1, true>(a, s);
      case 3 * 4 + 1: return retrieve_t<B, D, 3, 1, true>(a, s);
      case 1 * 4 + 2: return retrieve_t<B, D, 1, 2, true>(a, s);
      case 2 * 4 + 2: return retrieve_t<B, D, 2, 2, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
  switch (a.HP * 4 + KC) {
    case 1 * 4 + 1: return retrieve_t<B, D, 1, 1, false>(a, s);
    case 2 * 4 + 1: return retrieve_t<B, D, 2, 1, false>(a, s);
    case 3 * 4 + 1: return retrieve_t<B, D, 3, 1, false>(a, s);
    case 1 * 4 + 2: return retrieve_t<B, D, 1, 2, false>(a, s);
    case 2 * 4 + 2: return retrieve_t<B, D, 2, 2, false>(a, s);
    case 3 * 4 + 2: return retrieve_t<B, D, 3, 2, false>(a, s);
  }
  return hipErrorInvalidValue;
}

// Every slot of every wave holds a head, and the HP slots of each wave share one receiver and KV
// head: the kernel may then load one V tile set per wave with straight-line code.
static bool slots_fast(const RetrieveArgs& a) {
  for (int k = 0; k < a.n_split; ++k)
    for (int w = 0; w < 8; ++w)
      for (int j = w * a.HP; j < (w + 1) * a.HP; ++j) {
        if (a.slot_head[k][j] < 0) return false;
        if (a.slot_recv[k][j] != a.slot_recv[k][w * a.HP] || a.slot_kv[k][j] != a.slot_kv[k][w * a.HP]) return false;
      }
  return true;
}

hipError_t retrieve(const RetrieveArgs& a, hipStream_t s) {
  if (a.n_recv < 1 || a.n_recv > kMaxRecv || a.n_split < 1 || a.n_split > kMaxSplit || a.HP < 1 || a.HP > 4)
    return hipErrorInvalidValue;
  for (int k = 0; k < a.n_split; ++k) {
    const int n = a.split_nslots[k];
    if (n < 1 || n > 8 * a.HP) return hipErrorInvalidValue;
    for (int j = 0; j < 8 * a.HP; ++j) {
      // every slot, empty or not, names a receiver and one of its KV heads
      const int r = a.slot_recv[k][j], g = a.slot_head[k][j], kv = a.slot_kv[k][j];
      if ((j < n) != (g >= 0)) return hipErrorInvalidValue;
      if (r < 0 || r >= a.n_recv || kv < 0 || kv >= a.recv[r].H_kv || g >= a.recv[r].H_r)
        return hipErrorInvalidValue;
    }
  }
  RetrieveArgs b = a;
  b.fast = slots_fast(a) ? 1 : 0;
  if (a.B == 64 && a.d == 128) return retrieve_bd<64, 128>(b, s);
  if (a.B == 64 && a.d == 64) return retrieve_bd<64, 64>(b, s);
  if (a.B == 32 && a.d == 128) return retrieve_bd<32, 128>(b, s);
  if (a.B == 32 && a.d == 64) return retrieve_bd<32, 64>(b, s);
  return hipErrorInvalidValue;
}

}  // namespace mf
