// Host-only argument checks for the C ABI (no HIP calls, no device access).
#include "validate.hpp"

#include <cmath>
#include <cstdint>
#include <string>

namespace fa {
namespace {

int fail(std::string* msg, int status, const std::string& why) {
  if (msg) *msg = why;
  return status;
}

int check_mask_mod(const fa_mask_mod* mask, int32_t q_len, int32_t kv_len,
                   std::string* msg) {
  if (!mask) return fail(msg, FA_ERR_NULL_POINTER, "mask is NULL");
  switch (mask->kind) {
    case FA_MASK_NONE:
    case FA_MASK_CAUSAL:
      return FA_OK;
    case FA_MASK_SLIDING_WINDOW:
    case FA_MASK_LOCAL_WINDOW:
      if (mask->window < 1)
        return fail(msg, FA_ERR_INVALID_VALUE,
                    "window masks need window >= 1, got " +
                        std::to_string(mask->window));
      return FA_OK;
    case FA_MASK_DOCUMENT: {
      if (!mask->doc_id)
        return fail(msg, FA_ERR_NULL_POINTER, "document mask needs doc_id");
      int64_t need = q_len > kv_len ? q_len : kv_len;
      if (mask->doc_len < need)
        return fail(msg, FA_ERR_SHAPE_MISMATCH,
                    "doc_len " + std::to_string(mask->doc_len) +
                        " < max(q_len, kv_len) = " + std::to_string(need));
      if (mask->doc_stride < 0)
        return fail(msg, FA_ERR_INVALID_VALUE, "doc_stride must be >= 0");
      return FA_OK;
    }
    default:
      return fail(msg, FA_ERR_INVALID_VALUE,
                  "unknown mask kind " + std::to_string(mask->kind));
  }
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int check_strides(const char* name, const int64_t s[3], const int64_t dims[3],
                  int elt, std::string* msg) {
  if (!s) return fail(msg, FA_ERR_NULL_POINTER, std::string(name) + " stride is NULL");
  for (int d = 0; d < 3; ++d) {
    if (dims[d] <= 1) continue;
    if (s[d] < 0)
      return fail(msg, FA_ERR_INVALID_VALUE,
                  std::string(name) + " has a negative stride");
    if ((s[d] * elt) % 16 != 0)
      return fail(msg, FA_ERR_UNSUPPORTED,
                  std::string(name) + " stride " + std::to_string(d) + " = " +
                      std::to_string(s[d]) +
                      " elements is not a multiple of 16 bytes");
  }
  return FA_OK;
}

}  // namespace

int check_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t block_m,
                          int32_t block_n, int32_t* nqb, int32_t* nkvb,
                          std::string* msg) {
  if (!nqb || !nkvb)
    return fail(msg, FA_ERR_NULL_POINTER, "output pointer is NULL");
  if (q_len < 0 || kv_len < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative sequence length");
  if (block_m < 1 || block_n < 1)
    return fail(msg, FA_ERR_INVALID_VALUE, "block size must be >= 1");
  if (block_m > kMaxBlock || block_n > kMaxBlock)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "block size above " + std::to_string(kMaxBlock));
  int64_t q = (static_cast<int64_t>(q_len) + block_m - 1) / block_m;
  int64_t k = (static_cast<int64_t>(kv_len) + block_n - 1) / block_n;
  if (k > kMaxKvBlocks)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "more than " + std::to_string(kMaxKvBlocks) + " key blocks");
  *nqb = static_cast<int32_t>(q);
  *nkvb = static_cast<int32_t>(k);
  return FA_OK;
}

int check_create_block_mask(const fa_mask_mod* mask, int32_t B, int32_t H,
                            int32_t q_len, int32_t kv_len, int32_t block_m,
                            int32_t block_n, int32_t separate_full_blocks,
                            fa_block_mask* bm, BlockMaskLaunch* out,
                            std::string* msg) {
  if (!bm) return fail(msg, FA_ERR_NULL_POINTER, "bm is NULL");
  int st = check_mask_mod(mask, q_len, kv_len, msg);
  if (st != FA_OK) return st;
  if (B < 1 || H < 1)
    return fail(msg, FA_ERR_INVALID_VALUE, "B and H must be >= 1");
  int32_t nqb = 0, nkvb = 0;
  st = check_block_mask_dims(q_len, kv_len, block_m, block_n, &nqb, &nkvb, msg);
  if (st != FA_OK) return st;
  const bool sep = separate_full_blocks != 0;
  const int64_t rows = static_cast<int64_t>(B) * H * nqb;
  if (rows > INT32_MAX || rows * nkvb > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "B * H * num_q_blocks * num_kv_blocks too large");
  if (rows > 0) {
    if (!bm->kv_num_blocks)
      return fail(msg, FA_ERR_NULL_POINTER, "kv_num_blocks is NULL");
    if (nkvb > 0 && !bm->kv_indices)
      return fail(msg, FA_ERR_NULL_POINTER, "kv_indices is NULL");
    if (sep && !bm->full_kv_num_blocks)
      return fail(msg, FA_ERR_NULL_POINTER, "full_kv_num_blocks is NULL");
    if (sep && nkvb > 0 && !bm->full_kv_indices)
      return fail(msg, FA_ERR_NULL_POINTER, "full_kv_indices is NULL");
  }
  bm->mask = *mask;
  bm->B = B;
  bm->H = H;
  bm->q_len = q_len;
  bm->kv_len = kv_len;
  bm->block_m = block_m;
  bm->block_n = block_n;
  bm->num_q_blocks = nqb;
  bm->num_kv_blocks = nkvb;
  bm->separate_full_blocks = sep ? 1 : 0;
  if (!sep) {
    bm->full_kv_num_blocks = nullptr;
    bm->full_kv_indices = nullptr;
  }
  out->mask = MaskParams{mask->kind, mask->window, mask->doc_id,
                         mask->kind == FA_MASK_DOCUMENT ? mask->doc_stride : 0};
  out->Bm = B;
  out->Hm = H;
  out->q_len = q_len;
  out->kv_len = kv_len;
  out->block_m = block_m;
  out->block_n = block_n;
  out->nqb = nqb;
  out->nkvb = nkvb;
  out->separate_full = sep ? 1 : 0;
  out->num = bm->kv_num_blocks;
  out->idx = bm->kv_indices;
  out->fnum = bm->full_kv_num_blocks;
  out->fidx = bm->full_kv_indices;
  return FA_OK;
}

int check_flex_attention_fwd(int32_t dtype, int32_t B, int32_t H, int32_t H_kv,
                             int32_t q_len, int32_t kv_len, int32_t D,
                             const void* q, const int64_t q_stride[3],
                             const void* k, const int64_t k_stride[3],
                             const void* v, const int64_t v_stride[3],
                             float scale, const fa_block_mask* bm,
                             const fa_score_mod* score, void* o, float* lse,
                             FwdLaunch* out, bool* nothing_to_do,
                             std::string* msg) {
  *nothing_to_do = false;
  if (dtype != FA_BF16 && dtype != FA_FP32)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "unknown dtype " + std::to_string(dtype));
  if (B < 0 || H < 0 || q_len < 0 || kv_len < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative size");
  if (H_kv < 1 || H % H_kv != 0)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "H_kv must be >= 1 and divide H");
  if (D != 64 && D != 128)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "head dimension " + std::to_string(D) + " (built: 64, 128)");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(msg, FA_ERR_INVALID_VALUE, "scale must be finite and > 0");
  if (!bm) return fail(msg, FA_ERR_NULL_POINTER, "block mask is NULL");
  int st = check_mask_mod(&bm->mask, q_len, kv_len, msg);
  if (st != FA_OK) return st;
  if (bm->q_len != q_len || bm->kv_len != kv_len)
    return fail(msg, FA_ERR_SHAPE_MISMATCH,
                "block mask built for lengths (" + std::to_string(bm->q_len) +
                    ", " + std::to_string(bm->kv_len) + "), call has (" +
                    std::to_string(q_len) + ", " + std::to_string(kv_len) + ")");
  if (!(bm->B == 1 || bm->B == B) || !(bm->H == 1 || bm->H == H) ||
      bm->B < 1 || bm->H < 1)
    return fail(msg, FA_ERR_SHAPE_MISMATCH,
                "block mask batch/head dims must be 1 or equal to B/H");
  if (bm->mask.kind == FA_MASK_DOCUMENT && bm->mask.doc_stride != 0 && bm->B != B)
    return fail(msg, FA_ERR_SHAPE_MISMATCH,
                "per-batch document ids: the block mask must be built for B = " +
                    std::to_string(B) + " (it depends on the batch entry)");
  int32_t nqb = 0, nkvb = 0;
  st = check_block_mask_dims(q_len, kv_len, bm->block_m, bm->block_n, &nqb,
                             &nkvb, msg);
  if (st != FA_OK) return st;
  if (nqb != bm->num_q_blocks || nkvb != bm->num_kv_blocks)
    return fail(msg, FA_ERR_SHAPE_MISMATCH,
                "block mask block counts disagree with its lengths");
  const bool b64_128 = (bm->block_m == 64 || bm->block_m == 128) &&
                       (bm->block_n == 64 || bm->block_n == 128);
  if (!b64_128 || (dtype == FA_FP32 && bm->block_m != bm->block_n))
    return fail(msg, FA_ERR_UNSUPPORTED,
                "attention needs block_m, block_n in {64, 128} "
                "(and block_m == block_n for fp32)");
  int32_t skind = score ? score->kind : FA_SCORE_NONE;
  float cap = score ? score->softcap : 0.0f;
  if (skind != FA_SCORE_NONE && skind != FA_SCORE_SOFTCAP &&
      skind != FA_SCORE_ALIBI)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "unknown score kind " + std::to_string(skind));
  if (skind == FA_SCORE_SOFTCAP && (!std::isfinite(cap) || !(cap > 0.0f)))
    return fail(msg, FA_ERR_INVALID_VALUE, "softcap must be finite and > 0");
  const int64_t rows = static_cast<int64_t>(B) * H * nqb;
  if (rows > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED, "B * H * num_q_blocks too large");
  if (rows == 0) {
    *nothing_to_do = true;
    return FA_OK;
  }
  if (!q || !o) return fail(msg, FA_ERR_NULL_POINTER, "q or o is NULL");
  if (kv_len > 0 && (!k || !v))
    return fail(msg, FA_ERR_NULL_POINTER, "k or v is NULL");
  if (!bm->kv_num_blocks)
    return fail(msg, FA_ERR_NULL_POINTER, "kv_num_blocks is NULL");
  if (nkvb > 0 && !bm->kv_indices)
    return fail(msg, FA_ERR_NULL_POINTER, "kv_indices is NULL");
  if (bm->separate_full_blocks &&
      (!bm->full_kv_num_blocks || (nkvb > 0 && !bm->full_kv_indices)))
    return fail(msg, FA_ERR_NULL_POINTER, "full block arrays are NULL");
  const int elt = dtype == FA_BF16 ? 2 : 4;
  const int64_t qd[3] = {B, H, q_len};
  const int64_t kd[3] = {B, H_kv, kv_len};
  if ((st = check_strides("q", q_stride, qd, elt, msg)) != FA_OK) return st;
  if (kv_len > 0) {
    if ((st = check_strides("k", k_stride, kd, elt, msg)) != FA_OK) return st;
    if ((st = check_strides("v", v_stride, kd, elt, msg)) != FA_OK) return st;
  }
  // the bf16 kernels address a 64-row stage of K / V with 32-bit byte offsets
  if (kv_len > 0 && (k_stride[2] * elt * 64 >= (int64_t(1) << 31) ||
                     v_stride[2] * elt * 64 >= (int64_t(1) << 31)))
    return fail(msg, FA_ERR_UNSUPPORTED, "k / v sequence stride too large");
  if (!aligned16(q) || !aligned16(o) ||
      (kv_len > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(msg, FA_ERR_UNSUPPORTED, "q, k, v and o must be 16-byte aligned");

  out->B = B;
  out->H = H;
  out->H_kv = H_kv;
  out->q_len = q_len;
  out->kv_len = kv_len;
  out->D = D;
  out->q = q;
  out->k = k;
  out->v = v;
  for (int d = 0; d < 3; ++d) {
    out->qs[d] = q_stride[d];
    out->ks[d] = kv_len > 0 ? k_stride[d] : 0;
    out->vs[d] = kv_len > 0 ? v_stride[d] : 0;
  }
  out->scale = scale;
  out->mask = MaskParams{bm->mask.kind, bm->mask.window, bm->mask.doc_id,
                         bm->mask.kind == FA_MASK_DOCUMENT ? bm->mask.doc_stride : 0};
  out->Bm = bm->B;
  out->Hm = bm->H;
  out->block_m = bm->block_m;
  out->block_n = bm->block_n;
  out->nqb = nqb;
  out->nkvb = nkvb;
  out->num = bm->kv_num_blocks;
  out->idx = bm->kv_indices;
  out->fnum = bm->separate_full_blocks ? bm->full_kv_num_blocks : nullptr;
  out->fidx = bm->separate_full_blocks ? bm->full_kv_indices : nullptr;
  out->score_kind = skind;
  out->softcap = cap;
  out->o = o;
  out->lse = lse;
  out->nsplit = 1;
  out->part_o = nullptr;
  out->part_ml = nullptr;
  return FA_OK;
}

int check_split_workspace_bytes(int32_t B, int32_t H, int32_t q_len, int32_t D,
                                int32_t num_splits, uint64_t* bytes,
                                std::string* msg) {
  if (!bytes) return fail(msg, FA_ERR_NULL_POINTER, "bytes is NULL");
  if (B < 0 || H < 0 || q_len < 0 || D < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative size");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "num_splits must be in [1, " + std::to_string(kMaxSplits) + "]");
  if (num_splits == 1) {
    *bytes = 0;
    return FA_OK;
  }
  *bytes = static_cast<uint64_t>(num_splits) * static_cast<uint64_t>(B) *
           static_cast<uint64_t>(H) * static_cast<uint64_t>(q_len) *
           static_cast<uint64_t>(D + 2) * 4u;
  return FA_OK;
}

int check_fwd_workspace(int32_t dtype, void* workspace, uint64_t workspace_bytes,
                        FwdLaunch* p, std::string* msg) {
  p->sched = nullptr;
  if (!workspace) return FA_OK;
  if (!aligned16(workspace))
    return fail(msg, FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (workspace_bytes < FA_FWD_WORKSPACE_BYTES)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                    std::to_string(FA_FWD_WORKSPACE_BYTES));
  if (dtype == FA_BF16) p->sched = static_cast<unsigned int*>(workspace);
  return FA_OK;
}

int check_split(int32_t dtype, int32_t num_splits, void* workspace,
                uint64_t workspace_bytes, FwdLaunch* p, CombineLaunch* cl,
                std::string* msg) {
  uint64_t need = 0;
  int st = check_split_workspace_bytes(p->B, p->H, p->q_len, p->D, num_splits,
                                       &need, msg);
  if (st != FA_OK) return st;
  if (num_splits == 1) return FA_OK;
  if (dtype != FA_BF16)
    return fail(msg, FA_ERR_UNSUPPORTED, "split-KV is built for bf16 only");
  if (!workspace) return fail(msg, FA_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned16(workspace))
    return fail(msg, FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "workspace has " + std::to_string(workspace_bytes) +
                    " bytes, needs " + std::to_string(need));
  const int64_t rows = static_cast<int64_t>(p->B) * p->H * p->q_len;
  if (static_cast<int64_t>(p->B) * p->H * p->nqb * num_splits > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED, "too many split-KV workgroups");
  if (rows > INT32_MAX)  // the merge runs one workgroup per row
    return fail(msg, FA_ERR_UNSUPPORTED, "B * H * q_len too large for the split-KV merge");
  float* ws = static_cast<float*>(workspace);
  p->nsplit = num_splits;
  p->part_o = ws;
  p->part_ml = ws + static_cast<int64_t>(num_splits) * rows * p->D;
  cl->nsplit = num_splits;
  cl->rows = rows;
  cl->D = p->D;
  cl->part_o = p->part_o;
  cl->part_ml = p->part_ml;
  cl->o = p->o;
  cl->lse = p->lse;
  return FA_OK;
}

namespace {
uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }
}  // namespace

int bwd_workspace_layout(int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
                         int32_t kv_len, int32_t D, const fa_block_mask* bm,
                         int32_t num_splits, BwdWorkspace* ws, std::string* msg) {
  if (!bm || !ws) return fail(msg, FA_ERR_NULL_POINTER, "block mask or output is NULL");
  if (B < 0 || H < 0 || H_kv < 0 || q_len < 0 || kv_len < 0 || D < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative size");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "num_splits must be in [1, " + std::to_string(kMaxSplits) + "]");
  if (bm->B < 1 || bm->H < 1 || bm->num_q_blocks < 0 || bm->num_kv_blocks < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "block mask dims must be positive");
  const uint64_t rows = static_cast<uint64_t>(B) * static_cast<uint64_t>(H) *
                        static_cast<uint64_t>(q_len);
  const uint64_t bh = static_cast<uint64_t>(bm->B) * static_cast<uint64_t>(bm->H);
  const uint64_t nqb = static_cast<uint64_t>(bm->num_q_blocks);
  const uint64_t nkvb = static_cast<uint64_t>(bm->num_kv_blocks);
  const bool full = bm->separate_full_blocks != 0;
  uint64_t at = 0;
  ws->delta = at;
  at = align256(at + rows * 4u);
  ws->rowterm = at;
  at = align256(at + rows * 4u);
  ws->states = at;
  at = align256(at + bh * nqb * nkvb);
  ws->qnum = at;
  at = align256(at + bh * nkvb * 4u);
  ws->qidx = at;
  at = align256(at + bh * nkvb * nqb * 4u);
  ws->fqnum = at;
  at = full ? align256(at + bh * nkvb * 4u) : at;
  ws->fqidx = at;
  at = full ? align256(at + bh * nkvb * nqb * 4u) : at;
  // split mode: every part's fp32 sums of dQ, dK and dV
  const uint64_t parts = num_splits > 1 ? static_cast<uint64_t>(num_splits) : 0u;
  const uint64_t krows = static_cast<uint64_t>(B) * static_cast<uint64_t>(H_kv) *
                         static_cast<uint64_t>(kv_len);
  const uint64_t d = static_cast<uint64_t>(D);
  ws->part_dq = at;
  at = align256(at + parts * rows * d * 4u);
  ws->part_dk = at;
  at = align256(at + parts * krows * d * 4u);
  ws->part_dv = at;
  at = align256(at + parts * krows * d * 4u);
  ws->total = at;
  return FA_OK;
}

int check_flex_attention_bwd(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t dq_kv_order, int32_t num_splits,
    const void* o, const float* lse, const void* dout, void* workspace,
    uint64_t workspace_bytes, void* dq, void* dk, void* dv, BwdLaunch* out,
    bool* nothing_to_do, std::string* msg) {
  *nothing_to_do = false;
  if (dtype != FA_BF16)
    return fail(msg, FA_ERR_UNSUPPORTED, "the backward is built for bf16 only");
  if (dq_kv_order != 0 && dq_kv_order != 1)
    return fail(msg, FA_ERR_INVALID_VALUE, "dq_kv_order must be 0 or 1");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "num_splits must be in [1, " + std::to_string(kMaxSplits) + "]");
  // the forward's checks (o is only read here; the descriptor field is unused)
  int st = check_flex_attention_fwd(dtype, B, H, H_kv, q_len, kv_len, D, q,
                                    q_stride, k, k_stride, v, v_stride, scale,
                                    bm, score, const_cast<void*>(o),
                                    const_cast<float*>(lse), &out->f,
                                    nothing_to_do, msg);
  if (st != FA_OK) return st;
  out->zero_bytes = 0;
  if (*nothing_to_do) {
    // no query rows: with keys present, dK and dV are zero and still written
    const int64_t kv_elems = static_cast<int64_t>(B) * H_kv * kv_len * D;
    if (kv_elems == 0) return FA_OK;
    if (!dk || !dv) return fail(msg, FA_ERR_NULL_POINTER, "dk or dv is NULL");
    if (!aligned16(dk) || !aligned16(dv))
      return fail(msg, FA_ERR_UNSUPPORTED, "dk and dv must be 16-byte aligned");
    out->zero_bytes = static_cast<uint64_t>(kv_elems) * 2u;
    out->dk = dk;
    out->dv = dv;
    return FA_OK;
  }
  const int64_t kv_items = static_cast<int64_t>(B) * H_kv * bm->num_kv_blocks * num_splits;
  if (kv_items > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED, "B * H_kv * num_kv_blocks * num_splits too large");
  const int64_t q_items = static_cast<int64_t>(B) * H * bm->num_q_blocks * num_splits;
  if (q_items > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED, "B * H * num_q_blocks * num_splits too large");
  BwdWorkspace ws{};
  if ((st = bwd_workspace_layout(B, H, H_kv, q_len, kv_len, D, bm, num_splits, &ws, msg)) !=
      FA_OK)
    return st;
  if (!o || !lse || !dout || !dq)
    return fail(msg, FA_ERR_NULL_POINTER, "o, lse, dout or dq is NULL");
  if (kv_len > 0 && (!dk || !dv))
    return fail(msg, FA_ERR_NULL_POINTER, "dk or dv is NULL");
  if (ws.total > 0 && !workspace)
    return fail(msg, FA_ERR_NULL_POINTER, "workspace is NULL");
  if (workspace_bytes < ws.total)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "workspace has " + std::to_string(workspace_bytes) +
                    " bytes, needs " + std::to_string(ws.total));
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(lse) || (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return fail(msg, FA_ERR_UNSUPPORTED,
                "o, dout, dq, dk, dv and lse must be 16-byte aligned, the "
                "workspace 256-byte aligned");
  // the dK / dV kernel addresses a 64-row stage of Q with 32-bit byte offsets
  if (q_stride[2] * 2 * 64 >= (int64_t(1) << 31))
    return fail(msg, FA_ERR_UNSUPPORTED, "q sequence stride too large");
  char* w = static_cast<char*>(workspace);
  const bool full = bm->separate_full_blocks != 0;
  out->f.o = nullptr;
  out->f.lse = nullptr;
  out->o = o;
  out->lse = lse;
  out->dout = dout;
  out->delta = reinterpret_cast<float*>(w + ws.delta);
  out->rowterm = reinterpret_cast<float*>(w + ws.rowterm);
  out->states = reinterpret_cast<unsigned char*>(w + ws.states);
  out->qnum = reinterpret_cast<int32_t*>(w + ws.qnum);
  out->qidx = reinterpret_cast<int32_t*>(w + ws.qidx);
  out->fqnum = full ? reinterpret_cast<int32_t*>(w + ws.fqnum) : nullptr;
  out->fqidx = full ? reinterpret_cast<int32_t*>(w + ws.fqidx) : nullptr;
  out->dq = dq;
  out->dk = dk;
  out->dv = dv;
  out->dq_kv_order = dq_kv_order;
  out->f.nsplit = num_splits;
  out->kv_splits = num_splits;
  const bool split = num_splits > 1;
  out->part_dq = split ? reinterpret_cast<float*>(w + ws.part_dq) : nullptr;
  out->part_dk = split ? reinterpret_cast<float*>(w + ws.part_dk) : nullptr;
  out->part_dv = split ? reinterpret_cast<float*>(w + ws.part_dv) : nullptr;
  return FA_OK;
}

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
                       bool* nothing_to_do, std::string* msg) {
  *nothing_to_do = false;
  if (B < 0 || H < 0) return fail(msg, FA_ERR_INVALID_VALUE, "negative size");
  if (H_kv < 1 || H % H_kv != 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "H_kv must be >= 1 and divide H");
  if (H / H_kv > 32)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "decode packs a key head's query heads into 32 MFMA columns: "
                "H / H_kv must be <= 32");
  if (D != 64 && D != 128)
    return fail(msg, FA_ERR_UNSUPPORTED,
                "head dimension " + std::to_string(D) + " (built: 64, 128)");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(msg, FA_ERR_INVALID_VALUE, "scale must be finite and > 0");
  if (page_size < 64 || page_size % 64 != 0 || page_size > (1 << 20))
    return fail(msg, FA_ERR_UNSUPPORTED,
                "page_size must be a multiple of 64 in [64, 2^20]");
  if (max_pages < 0 || num_pages < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative page count");
  const int64_t cap = static_cast<int64_t>(max_pages) * page_size;
  if (cap > (int64_t(1) << 30))
    return fail(msg, FA_ERR_UNSUPPORTED, "max_pages * page_size above 2^30 tokens");
  if (!mask) return fail(msg, FA_ERR_NULL_POINTER, "mask is NULL");
  int st = check_mask_mod(mask, 0, static_cast<int32_t>(cap), msg);
  if (st != FA_OK) return st;
  int32_t skind = score ? score->kind : FA_SCORE_NONE;
  float softcap = score ? score->softcap : 0.0f;
  if (skind != FA_SCORE_NONE && skind != FA_SCORE_SOFTCAP && skind != FA_SCORE_ALIBI)
    return fail(msg, FA_ERR_INVALID_VALUE, "unknown score kind " + std::to_string(skind));
  if (skind == FA_SCORE_SOFTCAP && (!std::isfinite(softcap) || !(softcap > 0.0f)))
    return fail(msg, FA_ERR_INVALID_VALUE, "softcap must be finite and > 0");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(msg, FA_ERR_INVALID_VALUE,
                "num_splits must be in [1, " + std::to_string(kMaxSplits) + "]");
  const int64_t wgs = static_cast<int64_t>(B) * H_kv * num_splits;
  if (wgs > INT32_MAX || static_cast<int64_t>(B) * H > INT32_MAX)
    return fail(msg, FA_ERR_UNSUPPORTED, "too many workgroups");
  if (static_cast<int64_t>(B) * H == 0) {
    *nothing_to_do = true;
    return FA_OK;
  }
  if (!q || !o) return fail(msg, FA_ERR_NULL_POINTER, "q or o is NULL");
  if (!seq_lens) return fail(msg, FA_ERR_NULL_POINTER, "seq_lens is NULL");
  if (max_pages > 0 && (!page_table || !k_pages || !v_pages))
    return fail(msg, FA_ERR_NULL_POINTER, "page_table, k_pages or v_pages is NULL");
  if (max_pages > 0 && num_pages < 1)
    return fail(msg, FA_ERR_INVALID_VALUE, "num_pages must be >= 1");
  if (!q_stride || !k_stride || !v_stride)
    return fail(msg, FA_ERR_NULL_POINTER, "a stride array is NULL");
  for (int d = 0; d < 2; ++d)
    if (q_stride[d] < 0 || (q_stride[d] * 2) % 16 != 0)
      return fail(msg, FA_ERR_UNSUPPORTED, "q strides must be >= 0 and multiples of 16 bytes");
  for (int d = 0; d < 3; ++d)
    if (k_stride[d] < 0 || v_stride[d] < 0 || (k_stride[d] * 2) % 16 != 0 ||
        (v_stride[d] * 2) % 16 != 0)
      return fail(msg, FA_ERR_UNSUPPORTED,
                  "k / v page strides must be >= 0 and multiples of 16 bytes");
  // a 64-row stage is addressed with 32-bit byte offsets
  if (k_stride[1] * 2 * 64 >= (int64_t(1) << 31) || v_stride[1] * 2 * 64 >= (int64_t(1) << 31))
    return fail(msg, FA_ERR_UNSUPPORTED, "k / v row stride too large");
  if (!aligned16(q) || !aligned16(o) || (max_pages > 0 && (!aligned16(k_pages) || !aligned16(v_pages))))
    return fail(msg, FA_ERR_UNSUPPORTED, "q, o, k_pages and v_pages must be 16-byte aligned");
  uint64_t need = 0;
  if ((st = check_split_workspace_bytes(B, H, 1, D, num_splits, &need, msg)) != FA_OK) return st;
  if (num_splits > 1) {
    if (!workspace) return fail(msg, FA_ERR_NULL_POINTER, "workspace is NULL");
    if (!aligned16(workspace))
      return fail(msg, FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(msg, FA_ERR_INVALID_VALUE,
                  "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                      std::to_string(need));
  }
  out->B = B;
  out->H = H;
  out->H_kv = H_kv;
  out->D = D;
  out->q = q;
  out->qs[0] = q_stride[0];
  out->qs[1] = q_stride[1];
  out->k_pages = k_pages;
  out->v_pages = v_pages;
  for (int d = 0; d < 3; ++d) {
    out->ks[d] = k_stride[d];
    out->vs[d] = v_stride[d];
  }
  out->num_pages = num_pages;
  out->page_size = page_size;
  out->max_pages = max_pages;
  out->page_table = page_table;
  out->seq_lens = seq_lens;
  out->scale = scale;
  out->mask = MaskParams{mask->kind, mask->window, mask->doc_id,
                         mask->kind == FA_MASK_DOCUMENT ? mask->doc_stride : 0};
  out->score_kind = skind;
  out->softcap = softcap;
  out->nsplit = num_splits;
  out->o = o;
  out->lse = lse;
  const int64_t rows = static_cast<int64_t>(B) * H;
  float* ws = static_cast<float*>(workspace);
  out->part_o = num_splits > 1 ? ws : nullptr;
  out->part_ml = num_splits > 1 ? ws + static_cast<int64_t>(num_splits) * rows * D : nullptr;
  cl->nsplit = num_splits;
  cl->rows = rows;
  cl->D = D;
  cl->part_o = out->part_o;
  cl->part_ml = out->part_ml;
  cl->o = o;
  cl->lse = lse;
  return FA_OK;
}

int check_masked_softmax(int32_t BH, int32_t q_len, int32_t kv_len,
                         int64_t q_offset, const void* scores,
                         const int64_t score_stride[2],
                         const fa_mask_mod* mask, void* probs,
                         SoftmaxLaunch* out, bool* nothing_to_do,
                         std::string* msg) {
  *nothing_to_do = false;
  if (BH < 0 || q_len < 0 || kv_len < 0)
    return fail(msg, FA_ERR_INVALID_VALUE, "negative size");
  if (q_offset < 0 || q_offset > (int64_t(1) << 30))
    return fail(msg, FA_ERR_INVALID_VALUE, "q_offset must be in [0, 2^30]");
  if (kv_len % 8 != 0)
    return fail(msg, FA_ERR_UNSUPPORTED, "kv_len must be a multiple of 8 (16-byte rows)");
  if (!mask) return fail(msg, FA_ERR_NULL_POINTER, "mask is NULL");
  const int64_t qmax = q_offset + q_len;
  int st = check_mask_mod(mask, static_cast<int32_t>(qmax > INT32_MAX ? INT32_MAX : qmax),
                          kv_len, msg);
  if (st != FA_OK) return st;
  if (mask->kind == FA_MASK_DOCUMENT && mask->doc_stride != 0)
    return fail(msg, FA_ERR_UNSUPPORTED, "the masked softmax takes one shared doc_id array");
  if (mask->kind == FA_MASK_DOCUMENT && !aligned16(mask->doc_id))
    return fail(msg, FA_ERR_UNSUPPORTED, "doc_id must be 16-byte aligned");
  const int64_t rows = static_cast<int64_t>(BH) * q_len;
  if (rows == 0 || kv_len == 0) {
    *nothing_to_do = true;
    return FA_OK;
  }
  if (rows / 4 + 1 > INT32_MAX) return fail(msg, FA_ERR_UNSUPPORTED, "too many rows");
  if (!scores || !probs) return fail(msg, FA_ERR_NULL_POINTER, "scores or probs is NULL");
  if (!score_stride) return fail(msg, FA_ERR_NULL_POINTER, "score_stride is NULL");
  for (int d = 0; d < 2; ++d)
    if (score_stride[d] < 0 || (score_stride[d] * 2) % 16 != 0)
      return fail(msg, FA_ERR_UNSUPPORTED,
                  "score strides must be >= 0 and multiples of 16 bytes");
  if (!aligned16(scores) || !aligned16(probs))
    return fail(msg, FA_ERR_UNSUPPORTED, "scores and probs must be 16-byte aligned");
  out->rows = rows;
  out->q_len = q_len;
  out->kv_len = kv_len;
  out->q_offset = q_offset;
  out->scores = scores;
  out->ss[0] = score_stride[0];
  out->ss[1] = score_stride[1];
  out->mask = MaskParams{mask->kind, mask->window, mask->doc_id, 0};
  out->probs = probs;
  return FA_OK;
}

}  // namespace fa
