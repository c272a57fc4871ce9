/*
 * flexattn.h - C ABI of the MI355X (gfx950) block-sparse masked attention
 * library (libflexattn.so).
 *
 * FlexAttention-style operations:
 *
 *   fa_create_block_mask   turns a built-in mask_mod(b, h, q_idx, kv_idx)
 *                          into per-query-block lists of partial and full
 *                          key blocks ("How to Use FlexAttention on Apple
 *                          Silicon", sections "The two hooks" and
 *                          "Mask 1: causal"; tensorplay create_block_mask
 *                          page, parameters BLOCK_SIZE and
 *                          separate_full_blocks).
 *   fa_flex_attention_fwd  fused attention forward over such a block mask:
 *                          only live key blocks are read, mask_mod runs on
 *                          partial blocks only, score_mod runs on every
 *                          live position, and the softmax is computed online
 *                          so no score matrix is ever stored (how-to,
 *                          "The two hooks", "Bonus: a score_mod for
 *                          soft-capping"; frontiernews, "What Is
 *                          FlexAttention and Why Does It Matter").
 *   fa_flex_attention_bwd  its gradients dQ, dK, dV over the same block
 *                          mask (deterministic).
 *   fa_flex_attention_decode_paged  one decode step per sequence over a
 *                          paged key/value cache.
 *   fa_masked_softmax      the masked softmax of a materialising fallback,
 *                          mask folded into the score reads.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument named "device" is HIP device memory owned by
 *     the caller. The library never allocates, frees or synchronises; it
 *     enqueues kernels on the caller's HIP stream (hipStream_t passed as
 *     void*, NULL = the default stream) and returns.
 *   - Arguments are checked on the host before anything is enqueued. On any
 *     error nothing is launched and no output is written. A failed launch
 *     returns FA_ERR_HIP. Faults inside a kernel surface at the caller's
 *     next synchronisation, as for any HIP kernel.
 *   - fa_last_error() gives a human-readable reason for the most recent
 *     failure on the calling thread.
 *   - The functions keep no state between calls and may be called from
 *     several host threads.
 */
#ifndef FLEXATTN_H
#define FLEXATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 9

/* Bytes of the forward's scheduler workspace (see fa_flex_attention_fwd). */
#define FA_FWD_WORKSPACE_BYTES 256

/* Bytes of the fixed device scratch of fa_flex_attention_fwd_split_noalloc
 * (32 MiB per GPU the library runs on). */
#define FA_NOALLOC_SCRATCH_BYTES (32ull << 20)

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                 */
  FA_ERR_INVALID_VALUE = 2,  /* a value is out of its domain (W < 1, ...)  */
  FA_ERR_UNSUPPORTED = 3,    /* valid, but not built (dtype, D, block, ...) */
  FA_ERR_SHAPE_MISMATCH = 4, /* block mask and attention call disagree     */
  FA_ERR_HIP = 5             /* the HIP runtime refused a launch           */
} fa_status;

typedef enum fa_dtype { FA_BF16 = 0, FA_FP32 = 1 } fa_dtype;

/* Built-in mask_mods. True = the (query, key) pair is allowed.
 *   NONE            every pair ("either, both, or neither" hook may be
 *                   given: how-to, "The two hooks")
 *   CAUSAL          q_idx >= kv_idx (how-to, "Mask 1: causal")
 *   SLIDING_WINDOW  0 <= q_idx - kv_idx < window; the window counts the
 *                   diagonal (how-to, "Mask 2"; crackedaicode
 *                   "Sliding-Window Self-Attention", "State the boundary
 *                   precisely")
 *   DOCUMENT        q_idx >= kv_idx and doc_id[q_idx] == doc_id[kv_idx]
 *                   (how-to, "Mask 3: document-packed")
 *   LOCAL_WINDOW    |q_idx - kv_idx| < window: the symmetric local window,
 *                   limiting |i - j| instead of i - j (crackedaicode
 *                   "Sliding-Window Self-Attention", "State the boundary
 *                   precisely")
 * None of them depends on the batch or head index. */
typedef enum fa_mask_kind {
  FA_MASK_NONE = 0,
  FA_MASK_CAUSAL = 1,
  FA_MASK_SLIDING_WINDOW = 2,
  FA_MASK_DOCUMENT = 3,
  FA_MASK_LOCAL_WINDOW = 4
} fa_mask_kind;

/* Built-in score_mods, applied to the scaled score s = scale * q.k of
 * every live position (how-to, "The two hooks" and "Bonus"):
 *   NONE     s
 *   SOFTCAP  softcap * tanh(s / softcap)
 *   ALIBI    s - slope_h * (q_idx - kv_idx), slope_h = 2^(-8 (h + 1) / H),
 *            h = query head, H = number of query heads.
 * Accuracy of the bf16 forward's tanh: the exact form (a few float ulps of
 * 1); on a 64-key stage whose every |s / softcap| is at most 0.25, the odd
 * series to y^5 (error <= 3.3e-6), at most 0.15, to y^3 (<= 1.1e-5): below
 * the bf16 rounding of the softmax weights either way. */
typedef enum fa_score_kind {
  FA_SCORE_NONE = 0,
  FA_SCORE_SOFTCAP = 1,
  FA_SCORE_ALIBI = 2
} fa_score_kind;

typedef struct fa_mask_mod {
  int32_t kind;          /* fa_mask_kind                                  */
  int32_t window;        /* SLIDING_ / LOCAL_WINDOW: W >= 1; else ignored  */
  const int32_t* doc_id; /* DOCUMENT: device int32 [doc_len], indexed by
                            both q_idx and kv_idx; must outlive every use of
                            a block mask built from it. NULL otherwise.    */
  int64_t doc_len;       /* DOCUMENT: >= max(q_len, kv_len)                */
  int64_t doc_stride;    /* DOCUMENT: elements between the id arrays of
                            consecutive batch entries (a batch of packed
                            sequences: entry b reads doc_id + b * doc_stride);
                            0 = one array for every entry. With a stride the
                            mask depends on b: block masks are built with the
                            batch count (no broadcast over B).           */
} fa_mask_mod;

typedef struct fa_score_mod {
  int32_t kind;          /* fa_score_kind                                  */
  float softcap;         /* SOFTCAP: finite and > 0; ignored otherwise     */
} fa_score_mod;

/* A block mask. The index arrays are caller-allocated device memory of
 * int32; fa_create_block_mask fills them, fa_flex_attention_fwd reads them.
 *   kv_num_blocks       [B, H, NQB]         partial blocks per query block
 *                                           (every live block when
 *                                           separate_full_blocks == 0)
 *   kv_indices          [B, H, NQB, NKVB]   row m: the listed key blocks in
 *                                           ascending order, then all other
 *                                           key blocks in ascending order
 *                                           (each row is a permutation)
 *   full_kv_num_blocks  [B, H, NQB]         fully allowed blocks, on which
 *   full_kv_indices     [B, H, NQB, NKVB]   mask_mod is skipped; NULL when
 *                                           separate_full_blocks == 0
 * NQB = ceil(q_len / block_m), NKVB = ceil(kv_len / block_n). A block cut
 * by the end of a sequence is never full. B and H are 1 to broadcast one
 * mask over every batch entry / head (B=None, H=None on the how-to's
 * "Mask 1: causal"). The mask_mod is stored here: the attention call
 * applies it to partial blocks. */
typedef struct fa_block_mask {
  fa_mask_mod mask;
  int32_t B, H;
  int32_t q_len, kv_len;
  int32_t block_m, block_n;
  int32_t num_q_blocks, num_kv_blocks;
  int32_t separate_full_blocks;
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
} fa_block_mask;

/* Number of query and key blocks for the given lengths and block sizes.
 * q_len, kv_len >= 0; 1 <= block_m, block_n <= 1024. Host only. */
fa_status fa_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t block_m,
                             int32_t block_n, int32_t* num_q_blocks,
                             int32_t* num_kv_blocks);

/* create_block_mask (tensorplay create_block_mask page: the block mask is
 * derived from a mask_mod; separate_full_blocks has the meaning given
 * there).
 *
 * Classifies every (query block, key block) tile exactly over its in-range
 * (q_idx, kv_idx) pairs: no allowed pair = empty, all block_m * block_n
 * pairs allowed = full, otherwise partial (how-to, "The two mistakes": only
 * fully masked blocks are skipped). Then writes the index lists described at
 * fa_block_mask.
 *
 *   mask      host pointer; copied into bm->mask.
 *   B, H      1 = broadcast, else the batch / head count (>= 1).
 *   q_len, kv_len >= 0; 1 <= block_m, block_n <= 1024; NKVB <= 32768;
 *             B * H * NQB * NKVB < 2^31.
 *   bm        host pointer. In: the four device array pointers, sized as
 *             above (full_* may be NULL iff separate_full_blocks == 0).
 *             Out: every other field.
 *   stream    hipStream_t or NULL.
 * One kernel launch; asynchronous. */
fa_status fa_create_block_mask(const fa_mask_mod* mask, int32_t B, int32_t H,
                               int32_t q_len, int32_t kv_len, int32_t block_m,
                               int32_t block_n, int32_t separate_full_blocks,
                               fa_block_mask* bm, void* stream);

/* Fused block-sparse attention forward (flex_attention(q, k, v,
 * block_mask=, score_mod=) on the how-to's "Bonus" section; the shapes
 * follow scaled_dot_product_attention, how-to FAQ "What tensor shape does
 * flex_attention expect?").
 *
 *   dtype      FA_BF16 (bf16 inputs and O, fp32 accumulation) or FA_FP32.
 *   B, H       batch and query-head counts (>= 0; 0 is a no-op).
 *   H_kv       key/value heads, H % H_kv == 0; query head h reads key head
 *              h / (H / H_kv).
 *   q_len, kv_len  must equal bm->q_len, bm->kv_len.
 *   D          head dimension: 64 or 128.
 *   q          device [B, H, q_len, D] with element strides q_stride =
 *              {batch, head, sequence}; the D axis is contiguous.
 *   k, v       device [B, H_kv, kv_len, D], strides k_stride, v_stride.
 *              Every row start must be 16-byte aligned.
 *   scale      multiplies q.k before score_mod; finite and > 0
 *              (1/sqrt(D) is the usual choice).
 *   bm         host pointer to a block mask for (q_len, kv_len) with
 *              bm->B in {1, B}, bm->H in {1, H}, and block_m, block_n in
 *              {64, 128} (BLOCK_SIZE as an int or a (q, kv) pair, on the
 *              create_block_mask page; FA_FP32 needs block_m == block_n).
 *              Index arrays may come from
 *              fa_create_block_mask or from the caller; entries outside
 *              [0, NKVB) are skipped and counts are clamped to [0, NKVB].
 *              Caller lists must name each block of a row at most once,
 *              in the partial or in the full list, not both: a repeated
 *              entry is visited once per listing (its keys then count
 *              twice in the softmax), while the backward's transposed
 *              lists keep it once. Full blocks are taken as wholly
 *              allowed (mask_mod is not evaluated on them). With a
 *              per-batch doc_id (doc_stride != 0) the array must hold B
 *              rows of doc_len ids; the library cannot check this.
 *   score      host pointer to the score_mod (NULL = none).
 *   workspace  NULL, or device memory owned by the caller of at least
 *              FA_FWD_WORKSPACE_BYTES bytes, 16-byte aligned, all zero
 *              before its first use (workspace_bytes: its size). With a
 *              workspace the bf16 kernel keeps about two workgroups per
 *              compute unit resident and hands them query blocks one after
 *              another from counters kept there (the next block's first
 *              key/value tiles load while the current block finishes); the
 *              kernel leaves the counters zero again, so one workspace
 *              serves any number of calls in stream order. Calls in flight
 *              at the same time need separate workspaces. NULL: one
 *              workgroup per query block. Results are the same either way
 *              (same arithmetic per row). The fp32 instance ignores it.
 *   o          device [B, H, q_len, D], contiguous, dtype; 16-byte aligned.
 *   lse        device fp32 [B, H, q_len], contiguous; may be NULL.
 *              lse = ln sum_j exp(s_j) over the allowed keys of the row, in
 *              natural log; a row with no allowed key gets o = 0 and
 *              lse = -inf.
 *   stream     hipStream_t or NULL.
 * One kernel launch; asynchronous. */
fa_status fa_flex_attention_fwd(int32_t dtype, int32_t B, int32_t H,
                                int32_t H_kv, int32_t q_len, int32_t kv_len,
                                int32_t D, const void* q,
                                const int64_t q_stride[3], const void* k,
                                const int64_t k_stride[3], const void* v,
                                const int64_t v_stride[3], float scale,
                                const fa_block_mask* bm,
                                const fa_score_mod* score, void* workspace,
                                uint64_t workspace_bytes, void* o, float* lse,
                                void* stream);

/* Split-KV forward: the same operation as fa_flex_attention_fwd (same
 * arguments, results within rounding), executed with each query block's
 * list of live key blocks cut into num_splits consecutive parts that run as
 * separate workgroups. Each part keeps its own online softmax over its keys
 * and writes, per query row, the unnormalised output sum, the row maximum
 * and the row sum into `workspace`; a second kernel then merges the parts
 * exactly (the softmax over a union of disjoint key sets: rescale each part
 * by exp(m_part - m) and renormalise). This fills the GPU when B * H * NQB
 * is small against its 256 compute units, at the price of the partial
 * results' round trip through memory.
 *
 *   num_splits       1 ... 64. 1 is fa_flex_attention_fwd without a
 *                    scheduler workspace (workspace may be NULL). A part whose share of a row is empty writes a
 *                    neutral partial result.
 *   dtype            FA_BF16 when num_splits > 1 (else FA_ERR_UNSUPPORTED).
 *   workspace        device memory owned by the caller, 16-byte aligned, at
 *                    least fa_split_workspace_bytes(...) bytes; overwritten.
 *                    Calls in flight at the same time need separate
 *                    workspaces.
 *   workspace_bytes  its size; FA_ERR_INVALID_VALUE if too small.
 * Every other argument is as for fa_flex_attention_fwd. Two kernel
 * launches (num_splits > 1); asynchronous. */
fa_status fa_flex_attention_fwd_split(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t num_splits, void* workspace,
    uint64_t workspace_bytes, void* o, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as fa_flex_attention_fwd_split, with the parts' partial results
 * kept in a fixed scratch array of FA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on (from the first call on that GPU until the
 * process ends) instead of a caller workspace. No allocation of any kind.
 *
 *   num_splits  1 ... 64; the partial results must fit the scratch:
 *               fa_split_workspace_bytes(B, H, q_len, D, num_splits) <=
 *               FA_NOALLOC_SCRATCH_BYTES, else FA_ERR_INVALID_VALUE before
 *               anything is launched. 1 runs fa_flex_attention_fwd without a
 *               scheduler workspace (no scratch used).
 *   Every other argument is as for fa_flex_attention_fwd_split.
 * Calls on one GPU share its scratch: calls whose kernels may run at the
 * same time on one GPU (different streams, or different host threads) race
 * and give wrong results; serialise them. The scratch needs no clearing (each
 * part writes every row it owns before the merge reads it). Two kernel
 * launches (num_splits > 1); asynchronous. */
fa_status fa_flex_attention_fwd_split_noalloc(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t num_splits, void* o, float* lse,
    void* stream);

/* Workspace size of fa_flex_attention_fwd_split: num_splits * B * H * q_len
 * * (D + 2) * 4 bytes (fp32 partial outputs, then per-row maximum and
 * sum); 0 when num_splits == 1. Host only; nothing is launched.
 * FA_ERR_INVALID_VALUE for negative sizes or num_splits outside 1 ... 64. */
fa_status fa_split_workspace_bytes(int32_t B, int32_t H, int32_t q_len,
                                   int32_t D, int32_t num_splits,
                                   uint64_t* bytes);

/* Backward of fa_flex_attention_fwd (bf16): the gradients dQ, dK, dV of
 * o = attention(q, k, v) for an upstream gradient dout, over the same block
 * mask and score_mod (the lse output is not differentiated). The pages
 * presuppose this operation: the tensorplay create_block_mask page's
 * compute_dq_write_order / dq_kv_order parameters order the dQ writes of a
 * block-sparse backward over the block mask, and frontiernews ("What Else
 * Shipped in PyTorch 2.13?") lists a deterministic FlexAttention backward.
 * With t = scale q.k, s = score_mod(t), P = exp(s - lse) on allowed pairs
 * (0 elsewhere):
 *   dV = P^T dO,  dP = dO V^T,  delta_i = dO_i . O_i,
 *   dS = P * (dP - delta),  dT = dS * score_mod'(t)
 *        (1 for none and ALiBi, 1 - tanh^2(t / cap) for soft-cap),
 *   dQ = scale dT K,  dK = scale dT^T Q,
 * and with H_kv < H the gradients of a key head sum over its query heads.
 * Deterministic: no atomics; every output row is accumulated by one
 * workgroup in a fixed order, so repeated calls give identical bits. The
 * order of dQ's accumulation over key blocks is selectable, as with the
 * create_block_mask page's dq_kv_order (ascending or descending n-block
 * order); it changes only the rounding.
 *
 *   dtype      FA_BF16 only (FA_ERR_UNSUPPORTED otherwise).
 *   B ... score  as for fa_flex_attention_fwd (block_m, block_n in
 *              {64, 128}); bm and score must be the ones the forward ran
 *              with.
 *   dq_kv_order  0: each dQ row sums its live key blocks (partial and full
 *              lists merged by block index) in ascending block order; 1:
 *              descending, a block's later keys first. Other values:
 *              FA_ERR_INVALID_VALUE.
 *   num_splits 1 ... 64 (FA_ERR_INVALID_VALUE otherwise): 1 accumulates
 *              each gradient row in one workgroup. More cut each dQ row's
 *              and each dK / dV row's sequence of live blocks (in the
 *              order above) into num_splits consecutive parts of equal
 *              block count, run by separate workgroups, for grids too small
 *              to fill the GPU; each part's fp32 sum goes to the workspace
 *              and one more kernel adds the parts in part order, then
 *              scales and rounds. Still deterministic; the results differ
 *              from num_splits = 1 by rounding only.
 *   o          device bf16 [B, H, q_len, D], contiguous: the forward's output.
 *   lse        device fp32 [B, H, q_len], contiguous: the forward's lse.
 *              Gradients are only meaningful for the o and lse that the
 *              same arguments produced; other values give wrong numbers but
 *              no out-of-bounds access.
 *   dout       device bf16 [B, H, q_len, D], contiguous.
 *   workspace  device memory owned by the caller, 256-byte aligned, at
 *              least fa_bwd_workspace_bytes(...) bytes; overwritten. Calls in
 *              flight at the same time need separate workspaces.
 *   workspace_bytes  its size; FA_ERR_INVALID_VALUE if too small.
 *   dq         device bf16 [B, H, q_len, D], contiguous, written.
 *   dk, dv     device bf16 [B, H_kv, kv_len, D], contiguous, written (zero
 *              for keys that no allowed pair reaches).
 *   All device arrays 16-byte aligned; outputs must not overlap inputs.
 * Five kernel launches: three that transpose the block lists into
 * per-key-block lists of query blocks (clear, scatter, compact), the dQ
 * kernel (which also forms delta = rowsum(dO * O)), then the dK / dV
 * kernel, and with num_splits > 1 two that add the parts; asynchronous. */
fa_status fa_flex_attention_bwd(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t dq_kv_order, int32_t num_splits,
    const void* o, const float* lse, const void* dout, void* workspace,
    uint64_t workspace_bytes, void* dq, void* dk, void* dv, void* stream);

/* Workspace size of fa_flex_attention_bwd for a block mask: B * H * q_len
 * fp32 twice (delta and each row's exponent offset), then
 * bm->B * bm->H * NQB * NKVB bytes of tile states and the
 * transposed lists (per key block a count and NQB indices, int32, twice
 * when bm->separate_full_blocks), and with num_splits > 1 the parts' fp32
 * sums: num_splits * D * (B * H * q_len + 2 * B * H_kv * kv_len) * 4
 * bytes; each piece rounded up to 256 bytes. FA_ERR_INVALID_VALUE for
 * negative sizes or num_splits outside 1 ... 64. Host only (bm's dims are
 * read, not its arrays); nothing is launched. */
fa_status fa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t H_kv,
                                 int32_t q_len, int32_t kv_len, int32_t D,
                                 const fa_block_mask* bm, int32_t num_splits,
                                 uint64_t* bytes);

/* Decode step over a paged key/value cache (bf16). PagedAttention keeps the
 * key/value cache as pages, like virtual memory (frontiernews, "What
 * Attention Patterns Does FlexAttention Support?"); decoding runs one new
 * token per sequence under a causal or sliding-window mask (same section
 * and "What Are the Limitations of FlexAttention on Apple Silicon?").
 * Sequence b holds L_b = seq_lens[b] cached tokens, its newest token (whose
 * query is q[b]) included; token t of the sequence is row t % page_size of
 * physical page page_table[b * max_pages + t / page_size]. The query sits
 * at position q_idx = L_b - 1 and attends to keys kv_idx in [0, L_b) with
 * mask_mod(q_idx, kv_idx) and score_mod exactly as in fa_flex_attention_fwd
 * for that one row (ALiBi uses the query head h and these positions).
 *
 *   B, H, H_kv  sequences, query heads, key heads; H % H_kv == 0 and
 *              H / H_kv <= 32 (a key head's query heads share its tiles).
 *   D          64 or 128.
 *   q          device bf16 [B, H, D], element strides q_stride = {batch,
 *              head}; D contiguous; rows 16-byte aligned.
 *   k_pages, v_pages  device bf16 page pools: element (page, row, head, d)
 *              at page * stride[0] + row * stride[1] + head * stride[2] + d
 *              (e.g. [num_pages, page_size, H_kv, D] contiguous); strides
 *              multiples of 16 bytes.
 *   num_pages  pages in each pool (>= 1 when max_pages > 0).
 *   page_size  token rows per page: a multiple of 64 (no 64-key stage
 *              crosses a page).
 *   page_table device int32 [B, max_pages]. Entries for pages past L_b are
 *              never read; an entry outside [0, num_pages) is not read
 *              through either: its tokens are left out of the softmax.
 *   seq_lens   device int32 [B]; values are clamped to [0, max_pages *
 *              page_size]. L_b = 0 gives o = 0 and lse = -inf.
 *   scale      as for the forward.
 *   mask       host pointer: NONE, CAUSAL (both: every cached key),
 *              SLIDING_WINDOW or LOCAL_WINDOW (the last W keys) or
 *              DOCUMENT (keys of the query's document; doc_id indexed by
 *              token position, doc_len >= max_pages * page_size, doc_stride
 *              per sequence or 0).
 *   score      host pointer or NULL, as for the forward.
 *   num_splits 1 ... 64: each sequence's key range is cut into that many
 *              consecutive parts run as separate workgroups and merged
 *              exactly as in fa_flex_attention_fwd_split (workspace: at
 *              least fa_split_workspace_bytes(B, H, 1, D, num_splits)
 *              bytes, 16-byte aligned; NULL allowed for 1).
 *   o          device bf16 [B, H, D] contiguous; lse device fp32 [B, H] or
 *              NULL.
 * One or two kernel launches; asynchronous. */
fa_status fa_flex_attention_decode_paged(
    int32_t B, int32_t H, int32_t H_kv, int32_t D, const void* q,
    const int64_t q_stride[2], const void* k_pages, const int64_t k_stride[3],
    const void* v_pages, const int64_t v_stride[3], int32_t num_pages,
    int32_t page_size, const int32_t* page_table, int32_t max_pages,
    const int32_t* seq_lens, float scale, const fa_mask_mod* mask,
    const fa_score_mod* score, int32_t num_splits, void* workspace,
    uint64_t workspace_bytes, void* o, float* lse, void* stream);

/* Masked softmax over materialised scores (bf16 in and out, fp32 inside):
 * the compare / select-minimum / softmax chain of a materialising attention
 * fallback as one kernel (MLX pull request "Fuse the causal mask into the
 * SDPA fallback softmax"). For each of the BH * q_len rows, row i of a head
 * being query position q_idx = i + q_offset, and column j key position j:
 *   probs[row, j] = exp(s_j - m) / sum_{allowed} exp(s - m)  if
 *                   mask_mod(q_idx, j) allows the pair, else exactly 0,
 * m the maximum over the row's allowed scores; a row with no allowed key is
 * all zeros. Scores outside a row's allowed key interval are not read; no
 * mask or masked copy of the scores is written.
 *
 *   BH, q_len, kv_len  rows = BH * q_len; kv_len a multiple of 8.
 *   q_offset   >= 0: earlier tokens before the first row (a prefill chunk).
 *   scores     device bf16; row i of head slice b at b * score_stride[0] +
 *              i * score_stride[1] (elements, multiples of 8), columns
 *              contiguous; 16-byte aligned.
 *   mask       host pointer, any built-in kind (doc_id: one shared array,
 *              16-byte aligned, doc_len >= max(q_offset + q_len, kv_len)).
 *   probs      device bf16 [BH, q_len, kv_len] contiguous, 16-byte aligned.
 * One kernel launch; asynchronous. */
fa_status fa_masked_softmax(int32_t BH, int32_t q_len, int32_t kv_len,
                            int64_t q_offset, const void* scores,
                            const int64_t score_stride[2],
                            const fa_mask_mod* mask, void* probs,
                            void* stream);

/* Static description of a status code. */
const char* fa_status_string(int32_t status);

/* Reason for the most recent non-FA_OK return on this host thread. */
const char* fa_last_error(void);

/* FA_ABI_VERSION of the built library. */
int32_t fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLEXATTN_H */
