// create_block_mask on gfx950: exact tile classification, then per-row
// compaction with wavefront ballots and prefix counts.
//
// The block mask (tensorplay create_block_mask page, parameters BLOCK_SIZE
// and separate_full_blocks) records, for each query block m, which key blocks
// hold at least one allowed pair. Only fully masked blocks may be skipped
// (how-to "How to Use FlexAttention on Apple Silicon", "The two mistakes"),
// and fully allowed blocks can be listed apart so the attention kernel skips
// mask_mod on them (tensorplay page, separate_full_blocks).
//
// Two launches on the caller's stream:
//   classify_kernel  one wavefront per (query block, key block) tile. Each
//                    lane evaluates mask_mod on its columns for every row of
//                    the tile; the wave combines the per-pair results with
//                    ballots. Tile state (0 empty, 1 partial, 2 full) is
//                    written into kv_indices[.., m, n], which serves as the
//                    state array until the second launch overwrites it.
//   compact_kernel   one workgroup per query-block row. Loads the row's
//                    states into LDS, counts, then writes each index list as
//                    a stable partition (listed blocks ascending, then the
//                    rest ascending) using ballot + mbcnt prefix counts.
#include <hip/hip_runtime.h>

#include "../../include/flexattn.h"
#include "internal.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kEmpty = 0, kPartial = 1, kFull = 2;

// Evaluate the mask over one tile with one wavefront; returns the tile
// state, uniform across the wave.
template <int KIND>
__device__ int classify_tile(const MaskParams& mp, int i0, int rows, int j0,
                             int cols, int area, int lane) {
  bool any_true = false, any_false = false;
  const int* doc = mp.doc_id;
  for (int jc = 0; jc < cols; jc += 64) {
    const int jj = jc + lane;
    const bool in_range = jj < cols;
    const int j = j0 + (in_range ? jj : 0);
    int dj = 0;
    if (KIND == FA_MASK_DOCUMENT) dj = doc[j];
    for (int r = 0; r < rows; ++r) {
      const int i = i0 + r;
      bool ok;
      if (KIND == FA_MASK_NONE) {
        ok = true;
      } else if (KIND == FA_MASK_CAUSAL) {
        ok = i >= j;
      } else if (KIND == FA_MASK_SLIDING_WINDOW) {
        const int d = i - j;
        ok = (d >= 0) & (d < mp.window);
      } else {
        ok = (i >= j) & (doc[i] == dj);
      }
      const unsigned long long yes = __builtin_amdgcn_ballot_w64(in_range && ok);
      const unsigned long long no = __builtin_amdgcn_ballot_w64(in_range && !ok);
      any_true |= yes != 0ull;
      any_false |= no != 0ull;
      if (any_true && any_false) return kPartial;
    }
  }
  if (!any_true) return kEmpty;
  // every in-range pair allowed: full only if the tile is not cut short
  return (rows * cols == area) ? kFull : kPartial;
}

__global__ __launch_bounds__(kThreads) void classify_kernel(BlockMaskLaunch p,
                                                             int chunks) {
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int bid = blockIdx.x;
  const int chunk = bid % chunks;
  const int row = bid / chunks;            // (b, h, m) flattened
  const int m = row % p.nqb;
  const int n = chunk * kWaves + wave;
  if (n >= p.nkvb) return;
  const int i0 = m * p.block_m;
  const int j0 = n * p.block_n;
  const int rows = min(p.block_m, p.q_len - i0);
  const int cols = min(p.block_n, p.kv_len - j0);
  const int area = p.block_m * p.block_n;
  int state;
  switch (p.mask.kind) {
    case FA_MASK_CAUSAL:
      state = classify_tile<FA_MASK_CAUSAL>(p.mask, i0, rows, j0, cols, area, lane);
      break;
    case FA_MASK_SLIDING_WINDOW:
      state = classify_tile<FA_MASK_SLIDING_WINDOW>(p.mask, i0, rows, j0, cols, area, lane);
      break;
    case FA_MASK_DOCUMENT:
      state = classify_tile<FA_MASK_DOCUMENT>(p.mask, i0, rows, j0, cols, area, lane);
      break;
    default:
      state = classify_tile<FA_MASK_NONE>(p.mask, i0, rows, j0, cols, area, lane);
      break;
  }
  if (lane == 0) p.idx[static_cast<int64_t>(row) * p.nkvb + n] = state;
}

// Exclusive prefix count of `flag` over the workgroup for one chunk of
// kThreads consecutive key blocks; *chunk_total gets the chunk's count.
__device__ int wg_exclusive_count(bool flag, int* wave_counts, int* chunk_total) {
  const int wave = threadIdx.x / 64;
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(flag);
  const int lane_prefix = __builtin_amdgcn_mbcnt_hi(
      static_cast<unsigned>(mask >> 32),
      __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u));
  if ((threadIdx.x % 64) == 0) wave_counts[wave] = __builtin_popcountll(mask);
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int c = wave_counts[w];
    before += (w < wave) ? c : 0;
    total += c;
  }
  __syncthreads();  // wave_counts is reused by the next call
  *chunk_total = total;
  return before + lane_prefix;
}

__global__ __launch_bounds__(kThreads) void compact_kernel(BlockMaskLaunch p) {
  extern __shared__ unsigned char states[];   // nkvb bytes
  __shared__ int wave_counts[kWaves];
  __shared__ int totals[2];
  const int row = blockIdx.x;
  const int nkvb = p.nkvb;
  const bool sep = p.separate_full != 0;
  int32_t* idx = p.idx + static_cast<int64_t>(row) * nkvb;
  int32_t* fidx = sep ? p.fidx + static_cast<int64_t>(row) * nkvb : nullptr;

  if (threadIdx.x < 2) totals[threadIdx.x] = 0;
  int np = 0, nf = 0;
  for (int n = threadIdx.x; n < nkvb; n += kThreads) {
    const int s = idx[n];
    states[n] = static_cast<unsigned char>(s);
    np += sep ? (s == kPartial) : (s != kEmpty);
    nf += sep && (s == kFull);
  }
  __syncthreads();
  atomicAdd(&totals[0], np);
  atomicAdd(&totals[1], nf);
  __syncthreads();
  const int tot_p = totals[0];
  const int tot_f = totals[1];

  int run_p = 0, run_f = 0;
  for (int base = 0; base < nkvb; base += kThreads) {
    const int n = base + threadIdx.x;
    const bool in = n < nkvb;
    const int s = in ? states[n] : kEmpty;
    const bool is_p = in && (sep ? (s == kPartial) : (s != kEmpty));
    const bool is_f = in && sep && (s == kFull);
    int chunk_p, chunk_f;
    const int pp = run_p + wg_exclusive_count(is_p, wave_counts, &chunk_p);
    const int pf = run_f + wg_exclusive_count(is_f, wave_counts, &chunk_f);
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
  if (p.nkvb > 0) {
    const int chunks = (p.nkvb + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(classify_kernel, dim3(rows * chunks), dim3(kThreads), 0,
                       s, p, chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compact_kernel, dim3(rows), dim3(kThreads),
                     static_cast<size_t>(p.nkvb), s, p);
  return hipGetLastError();
}

}  // namespace fa
