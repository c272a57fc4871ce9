// Host-only argument checks for the C ABI. No HIP headers: this file and
// validate.cpp build with a plain C++ compiler.
#pragma once

#include <string>

#include "../../include/flexattn.h"
#include "internal.hpp"

namespace fa {

// Largest block size fa_create_block_mask accepts, and the largest number of
// key blocks per row (the builder keeps one byte per key block in LDS).
constexpr int kMaxBlock = 1024;
constexpr int kMaxKvBlocks = 32768;

int check_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t block_m,
                          int32_t block_n, int32_t* nqb, int32_t* nkvb,
                          std::string* msg);

// Fills *out for launch_block_mask and the output fields of *bm on success.
int check_create_block_mask(const fa_mask_mod* mask, int32_t B, int32_t H,
                            int32_t q_len, int32_t kv_len, int32_t block_m,
                            int32_t block_n, int32_t separate_full_blocks,
                            fa_block_mask* bm, BlockMaskLaunch* out,
                            std::string* msg);

// Fills *out for the forward launchers on success. *nothing_to_do is set when
// the problem is empty (B, H or q_len is 0): the call then succeeds without
// launching anything.
int check_flex_attention_fwd(int32_t dtype, int32_t B, int32_t H, int32_t H_kv,
                             int32_t q_len, int32_t kv_len, int32_t D,
                             const void* q, const int64_t q_stride[3],
                             const void* k, const int64_t k_stride[3],
                             const void* v, const int64_t v_stride[3],
                             float scale, const fa_block_mask* bm,
                             const fa_score_mod* score, void* o, float* lse,
                             FwdLaunch* out, bool* nothing_to_do,
                             std::string* msg);

// Largest number of split-KV parts per query block.
constexpr int kMaxSplits = 64;

// Sets the message fa_last_error() returns on the calling thread.
void record_error(const std::string& msg);

int check_split_workspace_bytes(int32_t B, int32_t H, int32_t q_len, int32_t D,
                                int32_t num_splits, uint64_t* bytes,
                                std::string* msg);

// Forward scheduler workspace: NULL (one workgroup per query block) or at
// least FA_FWD_WORKSPACE_BYTES, 16-byte aligned; sets p->sched for bf16.
int check_fwd_workspace(int32_t dtype, void* workspace, uint64_t workspace_bytes,
                        FwdLaunch* p, std::string* msg);

// Checks the split-KV arguments on top of a filled forward descriptor and
// sets its split fields (and *cl for the merge kernel).
int check_split(int32_t dtype, int32_t num_splits, void* workspace,
                uint64_t workspace_bytes, FwdLaunch* p, CombineLaunch* cl,
                std::string* msg);

// Backward workspace: delta and the exponent offsets (fp32 per query row),
// the tile-state matrix and the transposed block lists, each section
// 256-byte aligned.
struct BwdWorkspace {
  // byte offsets; part_* only with num_splits > 1
  uint64_t delta, rowterm, states, qnum, qidx, fqnum, fqidx, part_dq, part_dk, part_dv;
  uint64_t total;
};
int bwd_workspace_layout(int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
                         int32_t kv_len, int32_t D, const fa_block_mask* bm,
                         int32_t num_splits, BwdWorkspace* ws, std::string* msg);

// Fills *out for the backward launchers on success (the forward checks plus
// the backward's own restrictions). *nothing_to_do as for the forward.
int check_flex_attention_bwd(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t dq_kv_order, int32_t num_splits,
    const void* o, const float* lse, const void* dout, void* workspace,
    uint64_t workspace_bytes, void* dq, void* dk, void* dv, BwdLaunch* out,
    bool* nothing_to_do, std::string* msg);

// Fills *out for launch_decode_paged (and *cl for the merge when
// num_splits > 1) on success; *nothing_to_do when B * H == 0.
int check_decode_paged(int32_t B, int32_t H, int32_t H_kv, int32_t D,
                       const void* q, const int64_t q_stride[2],
                       const void* k_pages, const int64_t k_stride[3],
                       const void* v_pages, const int64_t v_stride[3],
                       int32_t num_pages, int32_t page_size,
                       const int32_t* page_table, int32_t max_pages,
                       const int32_t* seq_lens, float scale,
                       const fa_mask_mod* mask, const fa_score_mod* score,
                       int32_t num_splits, void* workspace,
                       uint64_t workspace_bytes, void* o, float* lse,
                       DecodeLaunch* out, CombineLaunch* cl,
                       bool* nothing_to_do, std::string* msg);

// Fills *out for launch_masked_softmax on success; *nothing_to_do when
// there is no row or no column.
int check_masked_softmax(int32_t BH, int32_t q_len, int32_t kv_len,
                         int64_t q_offset, const void* scores,
                         const int64_t score_stride[2],
                         const fa_mask_mod* mask, void* probs,
                         SoftmaxLaunch* out, bool* nothing_to_do,
                         std::string* msg);

}  // namespace fa
