// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

enum { DT_F32 = 0, DT_BF16 = 1 };

// kept blocks per gather work item.  Each item loads its block row's queries once, so longer
// items re-read them less; 128 measured fastest among 16 to 256 on an 8B->3B store at L = 32768.
constexpr int kGatherChunk = 128;

struct CompressArgs {
  const void* Q;
  const void* K;
  int dtype, H_s, d, B;
  int64_t T;
  int n_brow, nb_max;
  const int32_t* info;   // [n_brow][4]
  const int32_t* order;  // [n_brow]
  const int32_t* coff;   // [n_brow] causal block offset of each block row
  const int32_t* pairs;  // [n_pair][2] block rows (I, I+1) of one sequence, second may be -1
  int n_pair;
  const uint8_t* active; // [n_brow] rows to compress (NULL: all); order[] lists exactly these
  int n_order;           // entries of order[]
  int64_t n_causal;
  double tau;
  int options;           // MF_SELECT_PER_HEAD | MF_NORM_PER_HEAD (variants), 0 = the method as read
  uint8_t* hflags;       // [H_s][n_brow][nb_max] per-head kept flags (per-head selection)
  float* lse2n;          // [H_s][T] logsumexp plus log2 of the head's kept mass (per-head normalisation)
  float scale2;          // log2(e) / sqrt(d)
  // context scratch
  float2* zbuf;          // [H_s][n_causal][B] per (query, key block): {z, block max}
  float* lse2;           // [H_s][T]   log2-domain row logsumexp
  float* Mh;             // [H_s][n_brow][nb_max] per-head block masses
  double* M;             // [n_brow][nb_max] head-summed block masses
  uint8_t* flags;        // [n_brow][nb_max] kept flags
  int32_t* counts;       // [n_brow]
  double* part;          // [n_brow][ceil(nb_max / kGatherChunk)][H_s][B] row sums of stored probs per gather chunk
  void* ktile;           // [H_s][n_brow][B/16][fragment elements][64 lanes] key operands
  // fused prefill (attn_out != NULL): the statistics pass also writes the sender's own causal
  // attention output [T][H_s][d] fp32, from V prepared per sender head (fp16 tiles, exponents)
  const uint16_t* attn_vfrag;
  const int32_t* attn_vexps;
  float* attn_out;
  // the store
  int32_t* block_ptr;
  int32_t* block_idx;
  int32_t* block_row;
  uint16_t* probs;
  float* rkm;
  int32_t* counters;
  int64_t capacity;
};

// statistics, head reduction, selection and scan (writes block_ptr and counters)
hipError_t compress_plan(const CompressArgs& a, hipStream_t s);
// emit block indices, gather kept probabilities, kept row mass
hipError_t compress_fill(const CompressArgs& a, hipStream_t s);
bool compress_supported(int dtype, int B, int d);

struct VprepArgs {
  const void* V;
  int dtype, H_kv, d, B;
  int64_t T;
  int n_brow;
  const int32_t* info;
  const int32_t* page_table;  // NULL = contiguous
  int page_size, pages_per_seq;
  const int32_t* brow_seq;    // [n_brow] sequence of each block row (paged path)
  uint32_t* vmax_bits;        // [H_kv] scratch
  uint16_t* frag;
  int32_t* exps;
};
hipError_t v_prepare(const VprepArgs& a, hipStream_t s);

struct HeadMap {
  int8_t perm[64];  // receiver heads ordered by KV head
  int8_t kv[64];    // KV head of each receiver head
};

// One receiver of a (possibly fanned-out) retrieve.
struct RecvArgs {
  const float* W;        // [H_r][H_s]
  const uint16_t* vfrag; // prepared V tiles
  const int32_t* vexps;  // per-KV-head scale exponents
  float* O;              // [T][H_r][d]
  float* den;            // [T][H_r] running denominators (cross-layer accumulation), else NULL
  int H_r, H_kv;
};

constexpr int kMaxRecv = 4;    // receivers per fused retrieve
constexpr int kMaxSplit = 8;   // workgroups per row tile (head splits over all receivers)
constexpr int kMaxSlots = 32;  // slot-table entries per split (8 waves x 4)
constexpr int kSplitMax = 24;  // heads per split of the general schedule (8 waves x 3); 32 only for
                               // the half-block fast path of one grouped-query receiver

struct RetrieveArgs {
  const uint16_t* probs;
  const int32_t* block_ptr;
  const int32_t* block_idx;
  const int32_t* info;
  const int32_t* order;
  int64_t capacity;      // blocks allocated in the store (clamps block_ptr after an overflow)
  int n_brow, H_s, B, d;
  int n_order;           // block rows to retrieve: the first n_order entries of order[]
  int64_t T;
  const float* rkm;
  int n_recv, n_split;
  int accumulate;        // 0: normalised output; across sender layers 1: write the unnormalised
                         // output and denominator, 2: add to them, 3: add and normalise
  int HP;                                  // heads per wave (1..4): a split holds up to 8*HP heads
  int fast;                                // set by the launcher: straight-line fast path applies
  int8_t split_nslots[kMaxSplit];          // heads in each split; they fill its leading slots
  int8_t slot_recv[kMaxSplit][kMaxSlots];  // receiver of each slot
  int8_t slot_head[kMaxSplit][kMaxSlots];  // head within that receiver; -1 = empty
  int8_t slot_kv[kMaxSplit][kMaxSlots];    // KV head of that head
  RecvArgs recv[kMaxRecv];
};
hipError_t retrieve(const RetrieveArgs& a, hipStream_t s);
bool retrieve_supported(int B, int d, int H_r, int H_s);

struct DenseArgs {
  const void* Q;
  const void* K;
  int dtype, H_q, H_kv, d;
  int64_t T;
  int n_brow;            // 64-token block rows
  const int32_t* info;
  const int32_t* order;
  const int32_t* pairs;  // [n_pair][2] block rows (I, I+1) of one sequence, second may be -1
  int n_pair;
  const uint16_t* vfrag; // prepared V with B = 64
  const int32_t* vexps;
  HeadMap hm;
  float* O;
};
hipError_t dense_attention(const DenseArgs& a, hipStream_t s);
bool dense_supported(int dtype, int d);

hipError_t copy_probe(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t write_probe(void* dst, size_t bytes, const void* src, hipStream_t s);
hipError_t fill_probe(void* dst, size_t bytes, uint32_t v, hipStream_t s);

}  // namespace mf
