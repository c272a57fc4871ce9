// C-ABI entry points of libflexattn.so: check arguments on the host, pick the
// kernel instance, enqueue it on the caller's stream. No allocation, no
// synchronisation, no fallback path: anything not built is reported.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/flexattn.h"
#include "internal.hpp"
#include "validate.hpp"

namespace {

thread_local std::string g_last_error;

fa_status finish(int status, const std::string& msg) {
  if (status != FA_OK) g_last_error = msg;
  return static_cast<fa_status>(status);
}

fa_status hip_status(int err, const char* what) {
  if (err == 0) return FA_OK;
  g_last_error = std::string(what) + ": " +
                 hipGetErrorString(static_cast<hipError_t>(err));
  return FA_ERR_HIP;
}

}  // namespace

namespace fa {
void record_error(const std::string& msg) { g_last_error = msg; }
}  // namespace fa

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int32_t status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER";
    case FA_ERR_INVALID_VALUE: return "FA_ERR_INVALID_VALUE";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_SHAPE_MISMATCH: return "FA_ERR_SHAPE_MISMATCH";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "unknown fa_status";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t block_m,
                             int32_t block_n, int32_t* num_q_blocks,
                             int32_t* num_kv_blocks) {
  std::string msg;
  int st = fa::check_block_mask_dims(q_len, kv_len, block_m, block_n,
                                     num_q_blocks, num_kv_blocks, &msg);
  return finish(st, msg);
}

fa_status fa_create_block_mask(const fa_mask_mod* mask, int32_t B, int32_t H,
                               int32_t q_len, int32_t kv_len, int32_t block_m,
                               int32_t block_n, int32_t separate_full_blocks,
                               fa_block_mask* bm, void* stream) {
  std::string msg;
  fa::BlockMaskLaunch p{};
  int st = fa::check_create_block_mask(mask, B, H, q_len, kv_len, block_m,
                                       block_n, separate_full_blocks, bm, &p,
                                       &msg);
  if (st != FA_OK) return finish(st, msg);
  if (static_cast<int64_t>(p.Bm) * p.Hm * p.nqb == 0) return FA_OK;
  return hip_status(fa::launch_block_mask(p, stream), "block-mask kernel launch");
}

fa_status fa_flex_attention_fwd(int32_t dtype, int32_t B, int32_t H,
                                int32_t H_kv, int32_t q_len, int32_t kv_len,
                                int32_t D, const void* q,
                                const int64_t q_stride[3], const void* k,
                                const int64_t k_stride[3], const void* v,
                                const int64_t v_stride[3], float scale,
                                const fa_block_mask* bm,
                                const fa_score_mod* score, void* workspace,
                                uint64_t workspace_bytes, void* o, float* lse,
                                void* stream) {
  std::string msg;
  fa::FwdLaunch p{};
  bool nothing = false;
  int st = fa::check_flex_attention_fwd(dtype, B, H, H_kv, q_len, kv_len, D, q,
                                        q_stride, k, k_stride, v, v_stride,
                                        scale, bm, score, o, lse, &p, &nothing,
                                        &msg);
  if (st != FA_OK) return finish(st, msg);
  st = fa::check_fwd_workspace(dtype, workspace, workspace_bytes, &p, &msg);
  if (st != FA_OK) return finish(st, msg);
  if (nothing) return FA_OK;
  int err;
  if (dtype == FA_FP32)
    err = fa::launch_fwd_fp32(p, stream);
  else if (D == 64)
    err = fa::launch_fwd_bf16_d64(p, stream);
  else
    err = fa::launch_fwd_bf16_d128(p, stream);
  return hip_status(err, "attention kernel launch");
}

fa_status fa_split_workspace_bytes(int32_t B, int32_t H, int32_t q_len,
                                   int32_t D, int32_t num_splits,
                                   uint64_t* bytes) {
  std::string msg;
  return finish(fa::check_split_workspace_bytes(B, H, q_len, D, num_splits,
                                                bytes, &msg),
                msg);
}

fa_status fa_flex_attention_fwd_split(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t num_splits, void* workspace,
    uint64_t workspace_bytes, void* o, float* lse, void* stream) {
  std::string msg;
  fa::FwdLaunch p{};
  bool nothing = false;
  int st = fa::check_flex_attention_fwd(dtype, B, H, H_kv, q_len, kv_len, D, q,
                                        q_stride, k, k_stride, v, v_stride,
                                        scale, bm, score, o, lse, &p, &nothing,
                                        &msg);
  if (st != FA_OK) return finish(st, msg);
  fa::CombineLaunch cl{};
  st = fa::check_split(dtype, num_splits, workspace, workspace_bytes, &p, &cl,
                       &msg);
  if (st != FA_OK) return finish(st, msg);
  if (nothing) return FA_OK;
  int err;
  if (dtype == FA_FP32)
    err = fa::launch_fwd_fp32(p, stream);
  else if (D == 64)
    err = fa::launch_fwd_bf16_d64(p, stream);
  else
    err = fa::launch_fwd_bf16_d128(p, stream);
  if (err != 0 || p.nsplit == 1) return hip_status(err, "attention kernel launch");
  return hip_status(fa::launch_split_combine(cl, stream), "split-KV merge launch");
}

fa_status fa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t H_kv,
                                 int32_t q_len, int32_t kv_len, int32_t D,
                                 const fa_block_mask* bm, int32_t num_splits,
                                 uint64_t* bytes) {
  std::string msg;
  if (!bytes) return finish(FA_ERR_NULL_POINTER, "bytes is NULL");
  fa::BwdWorkspace ws{};
  int st = fa::bwd_workspace_layout(B, H, H_kv, q_len, kv_len, D, bm, num_splits, &ws, &msg);
  if (st != FA_OK) return finish(st, msg);
  *bytes = ws.total;
  return FA_OK;
}

fa_status fa_flex_attention_bwd(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t dq_kv_order, int32_t num_splits,
    const void* o, const float* lse, const void* dout, void* workspace,
    uint64_t workspace_bytes, void* dq, void* dk, void* dv, void* stream) {
  std::string msg;
  fa::BwdLaunch p{};
  bool nothing = false;
  int st = fa::check_flex_attention_bwd(
      dtype, B, H, H_kv, q_len, kv_len, D, q, q_stride, k, k_stride, v,
      v_stride, scale, bm, score, dq_kv_order, num_splits, o, lse, dout, workspace,
      workspace_bytes, dq, dk, dv, &p, &nothing, &msg);
  if (st != FA_OK) return finish(st, msg);
  if (nothing) {
    if (p.zero_bytes == 0) return FA_OK;
    int err = fa::launch_zero_fill(p.dk, p.zero_bytes, stream);
    if (err == 0) err = fa::launch_zero_fill(p.dv, p.zero_bytes, stream);
    return hip_status(err, "gradient clear launch");
  }
  int err = fa::launch_bwd_prepare(p, stream);
  if (err != 0) return hip_status(err, "backward preparation launch");
  err = D == 64 ? fa::launch_bwd_bf16_d64(p, stream) : fa::launch_bwd_bf16_d128(p, stream);
  if (err != 0 || p.kv_splits == 1) return hip_status(err, "attention backward launch");
  // split mode: the parts' sums, in part order
  const uint64_t q_elems = static_cast<uint64_t>(B) * H * q_len * D;
  const uint64_t kv_elems = static_cast<uint64_t>(B) * H_kv * kv_len * D;
  err = fa::launch_reduce_parts(p.part_dq, dq, p.f.scale, nullptr, nullptr, 0.0f, q_elems,
                                p.kv_splits, stream);
  if (err == 0)
    err = fa::launch_reduce_parts(p.part_dk, dk, p.f.scale, p.part_dv, dv, 1.0f, kv_elems,
                                  p.kv_splits, stream);
  return hip_status(err, "split backward merge launch");
}

fa_status fa_flex_attention_decode_paged(
    int32_t B, int32_t H, int32_t H_kv, int32_t D, const void* q,
    const int64_t q_stride[2], const void* k_pages, const int64_t k_stride[3],
    const void* v_pages, const int64_t v_stride[3], int32_t num_pages,
    int32_t page_size, const int32_t* page_table, int32_t max_pages,
    const int32_t* seq_lens, float scale, const fa_mask_mod* mask,
    const fa_score_mod* score, int32_t num_splits, void* workspace,
    uint64_t workspace_bytes, void* o, float* lse, void* stream) {
  std::string msg;
  fa::DecodeLaunch p{};
  fa::CombineLaunch cl{};
  bool nothing = false;
  int st = fa::check_decode_paged(B, H, H_kv, D, q, q_stride, k_pages, k_stride,
                                  v_pages, v_stride, num_pages, page_size,
                                  page_table, max_pages, seq_lens, scale, mask,
                                  score, num_splits, workspace, workspace_bytes,
                                  o, lse, &p, &cl, &nothing, &msg);
  if (st != FA_OK) return finish(st, msg);
  if (nothing) return FA_OK;
  int err = fa::launch_decode_paged(p, stream);
  if (err != 0 || p.nsplit == 1) return hip_status(err, "decode kernel launch");
  return hip_status(fa::launch_split_combine(cl, stream), "split-KV merge launch");
}

fa_status fa_masked_softmax(int32_t BH, int32_t q_len, int32_t kv_len,
                            int64_t q_offset, const void* scores,
                            const int64_t score_stride[2],
                            const fa_mask_mod* mask, void* probs,
                            void* stream) {
  std::string msg;
  fa::SoftmaxLaunch p{};
  bool nothing = false;
  int st = fa::check_masked_softmax(BH, q_len, kv_len, q_offset, scores,
                                    score_stride, mask, probs, &p, &nothing,
                                    &msg);
  if (st != FA_OK) return finish(st, msg);
  if (nothing) return FA_OK;
  return hip_status(fa::launch_masked_softmax(p, stream), "masked softmax launch");
}

}  // extern "C"
