// create_block_mask on gfx950: one kernel classifies every tile of a query
// block row exactly, then compacts the row's index lists with wavefront
// ballots and prefix counts.
//
// The block mask (tensorplay create_block_mask page, parameters BLOCK_SIZE
// and separate_full_blocks) records, for query block m, which key blocks hold
// at least one allowed pair. Only fully masked blocks may be skipped (how-to
// "How to Use FlexAttention on Apple Silicon", "The two mistakes"); fully
// allowed blocks are listed apart so the attention kernel skips mask_mod on
// them (tensorplay page, separate_full_blocks).
//
// Tile state over the in-range pairs (i, j) of a tile: no allowed pair =
// empty, every pair of a complete (uncut) tile allowed = full, else partial.
// How the kernel decides it, exactly, per mask kind:
//   * none, causal, sliding and local window: the predicate depends only on
//     d = i - j (an interval of allowed d),
//     and the pairs of a tile realise every integer d in
//     [i_lo - j_hi, i_hi - j_lo]. "Some pair allowed" and "all pairs allowed"
//     are therefore interval tests on that range (one thread per tile).
//   * document: a wavefront per tile. Pairs (i, j) allowed with document c
//     (doc[i] == doc[j] == c, i >= j) exist iff the query block's last row
//     of c is at or after the key block's first key of c; the tile is visited
//     one distinct key id at a time (one inside a document, two at a
//     boundary). All pairs are allowed iff both blocks are one and the same
//     document and the tile lies wholly below the diagonal. Ids need not be
//     sorted or contiguous. (Key blocks wider than 128 columns: a single-id
//     block takes the same test, a mixed one has every pair evaluated.)
// Compaction writes, per row, the listed blocks in ascending order followed by
// the remaining block numbers in ascending order (a stable partition).
#include <hip/hip_runtime.h>

#include <climits>

#include "../../include/flexattn.h"
#include "internal.hpp"

namespace fa {
namespace {

// Workgroup sizes: 16 waves for document masks (a wavefront per tile), 4 for
// the interval kinds (a thread per tile: a smaller group starts and passes
// its barriers sooner).
constexpr int kDocWaves = 16;
constexpr int kIntervalWaves = 4;
constexpr unsigned char kEmpty = 0, kPartial = 1, kFull = 2;

struct Tile {
  int i_lo, i_hi, j_lo, j_hi;  // inclusive in-range bounds
  bool complete;               // rows * cols == block area
};

__device__ __forceinline__ Tile make_tile(const BlockMaskLaunch& p, int m, int n) {
  Tile t;
  t.i_lo = m * p.block_m;
  t.i_hi = min(t.i_lo + p.block_m, p.q_len) - 1;
  t.j_lo = n * p.block_n;
  t.j_hi = min(t.j_lo + p.block_n, p.kv_len) - 1;
  t.complete = (t.i_hi - t.i_lo + 1) == p.block_m && (t.j_hi - t.j_lo + 1) == p.block_n;
  return t;
}

// d = i - j over the tile spans [dlo, dhi]; allowed d form [alo, ahi].
__device__ __forceinline__ unsigned char classify_range(const Tile& t, long long alo,
                                                        long long ahi) {
  const long long dlo = static_cast<long long>(t.i_lo) - t.j_hi;
  const long long dhi = static_cast<long long>(t.i_hi) - t.j_lo;
  if (dhi < alo || dlo > ahi) return kEmpty;
  if (dlo >= alo && dhi <= ahi && t.complete) return kFull;
  return kPartial;
}

__device__ __forceinline__ unsigned char classify_closed(const BlockMaskLaunch& p, int m, int n) {
  const Tile t = make_tile(p, m, n);
  switch (p.mask.kind) {
    case FA_MASK_CAUSAL:
      return classify_range(t, 0, 1LL << 40);
    case FA_MASK_SLIDING_WINDOW:
      return classify_range(t, 0, static_cast<long long>(p.mask.window) - 1);
    case FA_MASK_LOCAL_WINDOW:
      return classify_range(t, 1 - static_cast<long long>(p.mask.window),
                            static_cast<long long>(p.mask.window) - 1);
    default:  // none
      return t.complete ? kFull : kPartial;
  }
}

// Document mask, one wavefront per tile. `qdoc` holds the query block's
// document ids in LDS; `qsingle` is the id when the whole query block is one
// document, else INT_MIN.
__device__ unsigned char classify_document(const BlockMaskLaunch& p, const int* doc, int m,
                                           int n, const int* qdoc, int qsingle, int lane) {
  const Tile t = make_tile(p, m, n);
  const int cols = t.j_hi - t.j_lo + 1;
  const int rows = t.i_hi - t.i_lo + 1;
  // the query block's last row of document c (-1 if none)
  auto last_row_of = [&](int c) -> int {
    int last = -1;
    for (int base = 0; base < rows; base += 64) {
      const int r = base + lane;
      const unsigned long long hit =
          __builtin_amdgcn_ballot_w64(r < rows && qdoc[min(r, rows - 1)] == c);
      if (hit) last = t.i_lo + base + 63 - __builtin_clzll(hit);
    }
    return last;
  };
  if (cols <= 128) {
    // Allowed pairs with document c exist iff the query block's last row of
    // c is at or after the key block's first key of c, so the key block's
    // distinct ids are visited one at a time (one inside a document, two
    // at a boundary; ids need not be sorted): ids in two 64-column chunks,
    // `left*` the columns whose id is still to visit.
    const bool in0 = lane < cols, in1 = 64 + lane < cols;
    const int id0 = in0 ? doc[t.j_lo + lane] : 0;
    const int id1 = in1 ? doc[t.j_lo + 64 + lane] : 0;
    unsigned long long left0 = __builtin_amdgcn_ballot_w64(in0);
    unsigned long long left1 = __builtin_amdgcn_ballot_w64(in1);
    bool some = false;
    int distinct = 0, c_one = 0;
    while (left0 | left1) {
      const int c = left0 ? __builtin_amdgcn_readlane(id0, __builtin_ctzll(left0))
                          : __builtin_amdgcn_readlane(id1, __builtin_ctzll(left1));
      const unsigned long long h0 = __builtin_amdgcn_ballot_w64(in0 && id0 == c);
      const unsigned long long h1 = __builtin_amdgcn_ballot_w64(in1 && id1 == c);
      const int first_key = t.j_lo + (h0 ? __builtin_ctzll(h0) : 64 + __builtin_ctzll(h1));
      left0 &= ~h0;
      left1 &= ~h1;
      some |= last_row_of(c) >= first_key;
      ++distinct;
      c_one = c;
      if (some && distinct > 1) return kPartial;
    }
    if (!some) return kEmpty;
    // every pair allowed: one document on both sides and below the diagonal
    if (distinct == 1 && qsingle == c_one && t.i_lo >= t.j_hi && t.complete) return kFull;
    return kPartial;
  }
  // wider key blocks: is the key block a single document c?
  const int c = __builtin_amdgcn_readfirstlane(doc[t.j_lo]);
  bool other = false;
  for (int jj = lane; jj < cols; jj += 64) other |= doc[t.j_lo + jj] != c;
  if (!__builtin_amdgcn_ballot_w64(other)) {
    // pairs can only be allowed on rows of document c; (i, j) with i >= j
    // exists among them iff the last such row is >= the first key j_lo
    if (last_row_of(c) < t.j_lo) return kEmpty;
    // every pair allowed: one document on both sides and below the diagonal
    if (qsingle == c && t.i_lo >= t.j_hi && t.complete) return kFull;
    return kPartial;
  }
  // the key block mixes documents: evaluate every pair
  bool any_true = false, any_false = false;
  for (int jc = 0; jc < cols; jc += 64) {
    const int jj = jc + lane;
    const bool in = jj < cols;
    const int j = t.j_lo + (in ? jj : 0);
    const int dj = doc[j];
    for (int r = 0; r < rows; ++r) {
      const int i = t.i_lo + r;
      const bool ok = (i >= j) & (qdoc[r] == dj);
      any_true |= __builtin_amdgcn_ballot_w64(in && ok) != 0ull;
      any_false |= __builtin_amdgcn_ballot_w64(in && !ok) != 0ull;
      if (any_true && any_false) return kPartial;
    }
  }
  if (!any_true) return kEmpty;
  return t.complete ? kFull : kPartial;
}

// Exclusive prefix count of `flag` over the workgroup for one chunk of
// 64 kWaves consecutive key blocks; *chunk_total gets the chunk's count.
template <int kWaves>
__device__ int wg_exclusive_count(bool flag, int* wave_counts, int* chunk_total) {
  const int wave = threadIdx.x / 64;
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(flag);
  const int lane_prefix = __builtin_amdgcn_mbcnt_hi(
      static_cast<unsigned>(mask >> 32),
      __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u));
  if ((threadIdx.x % 64) == 0) wave_counts[wave] = __builtin_popcountll(mask);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = wave_counts[w];
    before += (w < wave) ? c : 0;
    total += c;
  }
  __syncthreads();  // wave_counts is reused by the next call
  *chunk_total = total;
  return before + lane_prefix;
}

template <int kWaves>
__global__ __launch_bounds__(64 * kWaves) void block_mask_kernel(BlockMaskLaunch p) {
  constexpr int kThreads = 64 * kWaves;
  extern __shared__ unsigned char states[];  // nkvb bytes
  __shared__ int wave_counts[kWaves];
  __shared__ int totals[2];
  __shared__ int qdoc[1024];  // document ids of the query block's rows
  const int row = blockIdx.x;  // (b, h, m) flattened
  const int m = row % p.nqb;
  const int nkvb = p.nkvb;
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const bool sep = p.separate_full != 0;

  // ---- classify
  if (p.mask.kind == FA_MASK_DOCUMENT) {
    const int i_lo = m * p.block_m;
    const int rows = min(i_lo + p.block_m, p.q_len) - i_lo;
    // this row's batch entry (rows are (b, h, m) flattened) and its ids
    const int b = row / (p.Hm * p.nqb);
    const int* doc = p.mask.doc_id + static_cast<int64_t>(b) * p.mask.doc_stride;
    for (int r = threadIdx.x; r < rows; r += kThreads) qdoc[r] = doc[i_lo + r];
    __syncthreads();
    const int first = qdoc[0];
    bool other = false;
    for (int r = threadIdx.x; r < rows; r += kThreads) other |= qdoc[r] != first;
    const int qsingle = __syncthreads_or(other) ? INT_MIN : first;
    for (int n = wave; n < nkvb; n += kWaves) {
      const unsigned char s = classify_document(p, doc, m, n, qdoc, qsingle, lane);
      if (lane == 0) states[n] = s;
    }
  } else {
    for (int n = threadIdx.x; n < nkvb; n += kThreads) states[n] = classify_closed(p, m, n);
  }
  if (threadIdx.x < 2) totals[threadIdx.x] = 0;
  __syncthreads();

  // ---- count, then compact as a stable partition
  int np = 0, nf = 0;
  for (int n = threadIdx.x; n < nkvb; n += kThreads) {
    const int s = states[n];
    np += sep ? (s == kPartial) : (s != kEmpty);
    nf += sep && (s == kFull);
  }
  atomicAdd(&totals[0], np);
  atomicAdd(&totals[1], nf);
  __syncthreads();
  const int tot_p = totals[0];
  const int tot_f = totals[1];

  int32_t* idx = p.idx + static_cast<int64_t>(row) * nkvb;
  int32_t* fidx = sep ? p.fidx + static_cast<int64_t>(row) * nkvb : nullptr;
  int run_p = 0, run_f = 0;
  for (int base = 0; base < nkvb; base += kThreads) {
    const int n = base + threadIdx.x;
    const bool in = n < nkvb;
    const int s = in ? states[n] : kEmpty;
    const bool is_p = in && (sep ? (s == kPartial) : (s != kEmpty));
    const bool is_f = in && sep && (s == kFull);
    int chunk_p, chunk_f;
    const int pp = run_p + wg_exclusive_count<kWaves>(is_p, wave_counts, &chunk_p);
    const int pf = run_f + wg_exclusive_count<kWaves>(is_f, wave_counts, &chunk_f);
    if (in) {
      idx[is_p ? pp : tot_p + (n - pp)] = n;
      if (sep) fidx[is_f ? pf : tot_f + (n - pf)] = n;
    }
    run_p += chunk_p;
    run_f += chunk_f;
  }
  if (threadIdx.x == 0) {
    p.num[row] = tot_p;
    if (sep) p.fnum[row] = tot_f;
  }
}

}  // namespace

int launch_block_mask(const BlockMaskLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rows = p.Bm * p.Hm * p.nqb;
  if (rows == 0) return hipSuccess;
  if (p.mask.kind == FA_MASK_DOCUMENT)
    hipLaunchKernelGGL(block_mask_kernel<kDocWaves>, dim3(rows), dim3(64 * kDocWaves),
                       static_cast<size_t>(p.nkvb), s, p);
  else
    hipLaunchKernelGGL(block_mask_kernel<kIntervalWaves>, dim3(rows), dim3(64 * kIntervalWaves),
                       static_cast<size_t>(p.nkvb), s, p);
  return hipGetLastError();
}

}  // namespace fa
