// Internal host-side launch descriptors shared by the C-ABI layer (api.cpp)
// and the kernel translation units. Plain data; no HIP types, so the
// argument checks in validate.cpp build with any C++ compiler.
#pragma once

#include <stdint.h>

namespace fa {

struct MaskParams {
  int32_t kind;           // fa_mask_kind
  int32_t window;         // sliding / local window W
  const int32_t* doc_id;  // device, document mask only
  int64_t doc_stride;     // elements between batch entries' ids (0: shared)
};

struct BlockMaskLaunch {
  MaskParams mask;
  int32_t Bm, Hm;
  int32_t q_len, kv_len;
  int32_t block_m, block_n;
  int32_t nqb, nkvb;
  int32_t separate_full;
  int32_t* num;
  int32_t* idx;
  int32_t* fnum;  // NULL when !separate_full
  int32_t* fidx;
};

struct FwdLaunch {
  int32_t B, H, H_kv;
  int32_t q_len, kv_len, D;
  const void* q;
  const void* k;
  const void* v;
  int64_t qs[3], ks[3], vs[3];  // element strides (batch, head, sequence)
  float scale;
  MaskParams mask;
  int32_t Bm, Hm;       // block-mask broadcast dims (1 or B / H)
  int32_t block_m;      // query rows per block
  int32_t block_n;      // keys per block
  int32_t nqb, nkvb;
  const int32_t* num;
  const int32_t* idx;
  const int32_t* fnum;  // may be NULL: no full blocks
  const int32_t* fidx;
  int32_t score_kind;
  float softcap;
  void* o;
  float* lse;           // may be NULL
  // split-KV: each query block's visit list is cut into nsplit consecutive
  // parts, one workgroup each (nsplit = 1: no split, o / lse written
  // directly). With nsplit > 1 the forward writes unnormalised partial
  // results (part_o [nsplit][B*H*q_len][D] fp32, part_ml [nsplit][B*H*q_len]
  // {row max in log2 units, row sum}) and a second kernel merges them.
  int32_t nsplit;
  float* part_o;
  float* part_ml;
  // persistent schedule (bf16, nsplit == 1): kSchedCounters zero-initialised
  // uint32 counters that the kernel leaves zero again; NULL = one workgroup
  // per item
  unsigned int* sched;
};

// Split-KV merge of the partial results described at FwdLaunch.
struct CombineLaunch {
  int32_t nsplit;
  int64_t rows;  // B * H * q_len
  int32_t D;
  const float* part_o;
  const float* part_ml;
  void* o;       // bf16 [rows][D]
  float* lse;    // may be NULL
};

// Backward: the forward's arguments (f: q, k, v, mask, block lists, score)
// plus the forward's outputs, the upstream gradient and the outputs.
struct BwdLaunch {
  FwdLaunch f;           // o / lse / split fields unused
  const void* o;         // forward output, [B, H, q_len, D] contiguous
  const float* lse;      // forward LSE, [B, H, q_len]
  const void* dout;      // dO, [B, H, q_len, D] contiguous
  float* delta;          // [B, H, q_len]: rowsum(dO * O), written by the dQ kernel
  // [B, H, q_len]: each row's exponent offset, -LSE log2(e) (minus the
  // ALiBi term slope_h log2(e) i), -inf for a row without keys; written by
  // the dQ kernel so that P = exp2(scale log2(e) q.k [+ slope log2(e) j] +
  // rowterm) in the dK / dV kernel
  float* rowterm;
  // per key block, the query blocks that list it ([Bm, Hm, nkvb] and
  // [Bm, Hm, nkvb, nqb]); full_* NULL when the mask has no full lists
  int32_t* qnum;
  int32_t* qidx;
  int32_t* fqnum;
  int32_t* fqidx;
  unsigned char* states; // [Bm, Hm, nqb, nkvb] scratch for the transposition
  void* dq;              // [B, H, q_len, D] contiguous, bf16
  void* dk;              // [B, H_kv, kv_len, D] contiguous, bf16
  void* dv;
  int32_t dq_kv_order;   // dQ accumulation over key blocks: 0 ascending, 1 descending
  // Split mode (kv_splits > 1, f.nsplit the same count): each key block's
  // visit sequence of the dK / dV kernel, and each query row's of the dQ
  // kernel, is cut into kv_splits parts run by separate workgroups; every
  // part writes its unscaled fp32 sums to part_* ([part][rows][D]), and
  // launch_reduce_parts adds them in part order. NULL when kv_splits == 1.
  int32_t kv_splits;
  float* part_dq;        // [kv_splits, B, H, q_len, D]
  float* part_dk;        // [kv_splits, B, H_kv, kv_len, D]
  float* part_dv;
  // no query rows (q_len == 0) but keys: bytes of dk and of dv to clear,
  // nothing else runs
  uint64_t zero_bytes;
};

// Decode step over a paged key/value cache: one query token per sequence
// at position seq_lens[b] - 1, keys [0, seq_lens[b]) read through the
// sequence's page table. Split into nsplit parts merged like the split-KV
// forward (part_o / part_ml layout of FwdLaunch with q_len = 1).
struct DecodeLaunch {
  int32_t B, H, H_kv, D;
  const void* q;                 // [B, H, D] bf16, strides qs (batch, head)
  int64_t qs[2];
  const void* k_pages;           // pool of pages, strides (page, row, head)
  const void* v_pages;
  int64_t ks[3], vs[3];
  int32_t num_pages, page_size, max_pages;
  const int32_t* page_table;     // [B, max_pages]
  const int32_t* seq_lens;       // [B]
  float scale;
  MaskParams mask;
  int32_t score_kind;
  float softcap;
  int32_t nsplit;
  void* o;                       // [B, H, D] bf16 contiguous
  float* lse;                    // [B, H] or NULL
  float* part_o;
  float* part_ml;
};

// Masked softmax over materialised scores: rows = (batch * head) * q_len
// rows of kv_len scores; row i of a head is query position i + q_offset.
struct SoftmaxLaunch {
  int64_t rows;
  int32_t q_len, kv_len;
  int64_t q_offset;
  const void* scores;   // bf16, element strides ss = (batch * head, row)
  int64_t ss[2];
  MaskParams mask;      // doc ids shared by every row (doc_stride 0)
  void* probs;          // bf16 [rows, kv_len] contiguous
};

// Kernel launchers: return a hipError_t value (0 = success).
int launch_block_mask(const BlockMaskLaunch& p, void* stream);
int launch_fwd_bf16_d64(const FwdLaunch& p, void* stream);
int launch_fwd_bf16_d128(const FwdLaunch& p, void* stream);
int launch_fwd_fp32(const FwdLaunch& p, void* stream);
int launch_split_combine(const CombineLaunch& p, void* stream);
int launch_bwd_prepare(const BwdLaunch& p, void* stream);  // transposed lists
// out_s = bf16(mul_s * sum over nsplit parts of parts_s), parts
// [nsplit][elems] fp32, added in part order; segment 1 optional (parts1
// NULL). elems a multiple of 8.
int launch_reduce_parts(const float* parts0, void* out0, float mul0, const float* parts1,
                        void* out1, float mul1, uint64_t elems, int nsplit, void* stream);
int launch_zero_fill(void* dst, uint64_t bytes, void* stream);  // 16-byte aligned
int launch_decode_paged(const DecodeLaunch& p, void* stream);
int launch_masked_softmax(const SoftmaxLaunch& p, void* stream);
int launch_bwd_bf16_d64(const BwdLaunch& p, void* stream);
int launch_bwd_bf16_d128(const BwdLaunch& p, void* stream);

}  // namespace fa
