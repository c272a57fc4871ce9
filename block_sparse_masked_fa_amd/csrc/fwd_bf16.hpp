// Fused block-sparse attention forward, bf16 inputs, fp32 accumulation, for
// gfx950 (MFMA v_mfma_f32_32x32x16_bf16, LDS DMA, transposed LDS reads).
//
// Work split. One workgroup computes one query block (BQ = 64 or 128 rows)
// of one head with BQ / 32 wavefronts; wave w owns query rows
// [32w, 32w + 32). Key blocks (BK = 64 or 128 keys) are consumed in stages
// of 64 keys. Two workgroups share a CU (registers <= 256 per lane, 64 KB of LDS each at
// D = 128), so while one is in its MFMA phase the other's softmax arithmetic
// can issue: the two are independent and drift apart.
//
// Block order. A row's live key blocks are visited partial list first, then
// the full list, each from the last block to the first, and the stages of a
// block from its last keys to its first. Under causal-style masks (the
// diagonal block is the last partial one) this visits the keys nearest the
// query first; with a distance penalty (ALiBi) the running maximum is then
// found early and later stages rarely raise it, so the output accumulator is
// rarely rescaled.
//
// Data movement. For each stage the K and V tiles [64 keys][D] go HBM -> LDS
// with buffer loads that write LDS directly (no register staging; issued as
// inline asm, see fwd_asm.hpp), double-buffered so the next stage is in
// flight while this one is computed. Each tile is read through a buffer
// descriptor that ends at the sequence end, so rows past it arrive as zeros.
// In LDS a tile is row-major with its 16-byte chunks XOR-swizzled per row;
// the swizzle makes both read patterns conflict-free on the 64 LDS banks:
//   * S^T = K Q^T takes K as the MFMA A operand: ds_read_b128, 16 rows x one
//     chunk per 16 lanes;
//   * O^T += V^T P^T needs V with keys along each lane's k slots:
//     ds_read_b64_tr_b16 transposes on the fly from the row-major tile
//     (4 rows x 4 chunks per 32 lanes).
// Q^T is the B operand of S^T for the whole row and stays in registers. With
// keys on the MFMA row axis, every accumulator value of a lane belongs to the
// same query (column lane % 32), so row reductions are in-lane plus one
// exchange with lane ^ 32, and P leaves the accumulator already laid out as
// the B operand of the PV product (the MFMA contracts over its k slots in any
// order that A and B agree on; the transposed V reads follow that order).
//
// Online softmax (log2 domain, exp2 on v_exp_f32). Per stage: s2 = score_mod
// (scale * q.k) * log2(e); mask_mod on partial / sequence-tail blocks only;
// row max; p = exp2(s2 - m_ref). The reference m_ref is raised only when the
// row max exceeds it by more than kRescaleSlack (then l and the accumulator
// are multiplied by exp2(m_old - m_new)); otherwise p may exceed 1 by at most
// 2^kRescaleSlack, which fp32 and bf16 represent with the same relative
// precision. The row sum adds the bf16-rounded p (v_dot2c_f32_bf16 against
// ones), i.e. exactly the weights the PV product uses. Soft-capped scores are
// bounded by the cap, so for caps up to kCapFixedRefMax the reference is a
// constant set from the cap alone and the stages take no row max at all.
#pragma once

#include "fwd_asm.hpp"
#include "fwd_common.hpp"

namespace fa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlack = 8.0f;
// Soft-capped scores lie in [-capL, capL] (capL = cap log2 e, log2 units).
// Against the fixed reference m_ref = capL - kCapHeadroom every weight
// p = exp2(s2 - m_ref) lies in [2^(kCapHeadroom - 2 capL), 2^kCapHeadroom];
// while capL <= kCapFixedRefMax that is inside [2^-112, 2^48]: no weight
// overflows or leaves the normal range (fp32 and bf16 alike), the row sum
// and the accumulator stay below 2^79 |v|max for rows up to 2^31 keys, and
// the stage loop needs neither a row maximum nor a rescale.
constexpr float kCapHeadroom = 48.0f;
constexpr float kCapFixedRefMax = 80.0f;
// A soft-cap stage whose every |y| = |q.k scale / cap| is at most
// kCapSeriesY takes cap tanh y from its odd series to y^5,
// y - y^3 / 3 + 2 y^5 / 15: the series alternates with falling terms there,
// so the error is below the first omitted one, 17 y^7 / 315 <= 3.3e-6 (of
// the cap), against 2^-9 for the bf16 rounding of every weight. Up to
// kCapSeries3Y the series stops at y^3, error below 2 y^5 / 15 <= 1.1e-5
// (of the cap; 5.1e-4 at cap 50, a relative 5.1e-4 on a weight, a quarter
// of its bf16 rounding), one FMA fewer per score.
constexpr float kCapSeriesY = 0.25f;
constexpr float kCapSeries3Y = 0.15f;
constexpr int kStageKeys = 64;
constexpr int kSReadAhead = 6;  // K operand reads in flight ahead of the S product

template <int D>
__device__ __forceinline__ int kv_swizzle(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

// max / sum of x over lanes l and l ^ 32 (the two halves of a query row's
// keys): v_permlane32_swap exchanges the upper half of one register with the
// lower half of another, so after swapping two copies of x each lane holds
// x[l] and x[l ^ 32]. No LDS round trip, unlike a generic shuffle.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float row_pair_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float row_pair_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

// The kernel's FwdLaunch argument read straight from the kernel argument
// segment (it is the only argument, at offset 0) through a pointer the
// compiler cannot see through: every use is a fresh scalar load (a scalar
// cache hit) instead of a value held in scalar registers for the whole
// kernel. Used for the fields a persistent workgroup needs only at item
// boundaries.
typedef const __attribute__((address_space(4))) FwdLaunch KArgs;
__device__ __forceinline__ KArgs& kargs() {
  KArgs* q = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(q));
  return *q;
}

// Logical item -> (head, query block, split part). Logical items are dealt
// to the 8 XCDs in contiguous ranges (workgroups are dispatched round-robin,
// wg % 8, so the range of XCD x is served by workgroups x, x + 8, ...): the
// query blocks of one head run on one XCD and share its L2. Within a head the
// heaviest query blocks (last rows under causal masks) come first.
template <class Params>
__device__ __forceinline__ bool logical_item(const Params& p, int logical, WorkItem& w) {
  const int total = p.B * p.H * p.nqb * p.nsplit;
  if (logical < 0 || logical >= total) return false;
  w.c = logical % p.nsplit;  // the parts of one query block run side by side
  const int row = logical / p.nsplit;
  w.m = p.nqb - 1 - (row % p.nqb);
  const int bh = row / p.nqb;
  w.h = bh % p.H;
  w.b = bh / p.H;
  return true;
}

// One workgroup per item: workgroup wg serves slot wg / 8 of XCD wg % 8.
__device__ __forceinline__ bool xcd_work_item(const FwdLaunch& p, WorkItem& w) {
  const int total = p.B * p.H * p.nqb * p.nsplit;
  const int per_xcd = (total + 7) >> 3;
  const int wg = blockIdx.x;
  return logical_item(p, (wg & 7) * per_xcd + (wg >> 3), w);
}

// Persistent schedule (p.sched != NULL): gridDim.x workgroups (a multiple of
// 8, about two per compute unit) stay resident and take items one after
// another. Slot j of XCD x first takes the j-th item of its XCD's range; after
// that each XCD's range is handed out by its own counter, sched[x] (item
// slots + the counter's old value), and a workgroup whose range is used up
// takes items from the following XCDs' ranges. A workgroup that finds every
// range used up adds one to sched[8]; the last one to do so puts all nine
// counters back to zero, so the array is zero again for the next launch.
// Returns the logical item, or -1 when no range has an item left.
constexpr int kSchedCounters = 9;
static_assert(kSchedCounters * 4 <= FA_FWD_WORKSPACE_BYTES, "scheduler counters fit the workspace");

// Launch shape (host): a persistent grid of two workgroups per compute unit
// when the launch has scheduler counters and more items than that; else one
// workgroup per item (counters dropped), rounded up to whole XCD rounds.
inline FwdLaunch fwd_schedule(const FwdLaunch& p, int items, unsigned* wgs) {
  FwdLaunch q = p;
  int dev = 0, cus = 0;
  if (q.sched && hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0) {
    const int slots = (2 * cus + 7) / 8 * 8;
    if (items > slots) {
      *wgs = static_cast<unsigned>(slots);
      return q;
    }
  }
  q.sched = nullptr;
  *wgs = static_cast<unsigned>((items + 7) / 8 * 8);
  return q;
}

// The item a counter value `got` from XCD range xs names, or -2 when that
// range is used up (no atomics: usable inside the stage loop).
template <class Params>
__device__ __forceinline__ int sched_check(const Params& p, unsigned got, int xs) {
  const int total = p.B * p.H * p.nqb * p.nsplit;
  const int per_xcd = (total + 7) >> 3;
  const int slots = static_cast<int>(gridDim.x >> 3);
  const int64_t k = static_cast<int64_t>(got) + slots;
  const int64_t logical = static_cast<int64_t>(xs & 7) * per_xcd + k;
  return k < per_xcd && logical < total ? static_cast<int>(logical) : -2;
}

template <class Params>
__device__ __forceinline__ int sched_resolve(const Params& p, unsigned got, int& xs) {
  const int total = p.B * p.H * p.nqb * p.nsplit;
  const int per_xcd = (total + 7) >> 3;
  const int slots = static_cast<int>(gridDim.x >> 3);
  const int x0 = static_cast<int>(blockIdx.x & 7);
  for (;;) {
    const int x = xs & 7;
    const int64_t k = static_cast<int64_t>(got) + slots;
    const int64_t logical = static_cast<int64_t>(x) * per_xcd + k;
    if (k < per_xcd && logical < total) return static_cast<int>(logical);
    if (++xs >= x0 + 8) return -1;
    got = __hip_atomic_fetch_add(p.sched + (xs & 7), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void sched_finish(const FwdLaunch& p) {
  const unsigned n = __hip_atomic_fetch_add(p.sched + 8, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  if (n == gridDim.x - 1) {
    for (int c = 0; c < kSchedCounters; ++c)
      __hip_atomic_store(p.sched + c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// DOC: the document mask (per-key document ids staged in LDS and compared on
// partial blocks); every other built-in mask is an interval test only.
template <int D, int BQ, int BK, int SCORE, bool DOC>
__global__ __launch_bounds__(BQ * 2, 2) void fwd_bf16_kernel(const FwdLaunch p) {
  constexpr int NW = BQ / 32;             // wavefronts
  constexpr int NT = NW * 64;             // threads
  constexpr int SPB = BK / kStageKeys;    // stages per key block
  constexpr int RB = D * 2;               // bytes per LDS row
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPK = 1024 / RB;          // rows per 1 KB DMA segment
  constexpr int STAGE_BYTES = kStageKeys * RB;
  constexpr int ROUNDS = STAGE_BYTES / (NT * 16);
  constexpr int DK = D / 16;
  constexpr int DT = D / 32;

  // LDS: two stage buffers (K and V tiles), their document ids, and the
  // persistent schedule's next item (-1 for none), in one array so that
  // every address is one base plus a constant
  constexpr int OFF_DOC = 4 * STAGE_BYTES;
  constexpr int OFF_NEXT = OFF_DOC + 2 * kStageKeys * 4;
  __shared__ __attribute__((aligned(1024))) char smem[OFF_NEXT + 16];
  char* const sK0 = smem;
  char* const sV0 = smem + STAGE_BYTES;
  char* const sK1 = smem + 2 * STAGE_BYTES;
  char* const sV1 = smem + 3 * STAGE_BYTES;
  int* const sDoc0 = reinterpret_cast<int*>(smem + OFF_DOC);
  int* const sDoc1 = reinterpret_cast<int*>(smem + OFF_DOC + kStageKeys * 4);
  int& sNext = *reinterpret_cast<int*>(smem + OFF_NEXT);

  const bool persistent = p.sched != nullptr;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  // ---- the first item
  WorkItem w;
  int xs = static_cast<int>(blockIdx.x & 7);  // XCD range being drained
  bool have;
  if (!persistent) {
    have = xcd_work_item(p, w);
  } else {
    const int total = p.B * p.H * p.nqb * p.nsplit;
    const int per_xcd = (total + 7) >> 3;
    const int j = static_cast<int>(blockIdx.x >> 3);
    int first = j < per_xcd ? xs * per_xcd + j : total;
    if (first >= total) {
      // this slot's static item is past its XCD's range: take one from the
      // counters (the same for every wave: one lane asks, LDS broadcasts)
      if (tid == 0) {
        const unsigned got = __hip_atomic_fetch_add(p.sched + xs, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        sNext = sched_resolve(p, got, xs);
      }
      __syncthreads();
      first = __builtin_amdgcn_readfirstlane(sNext);
      __syncthreads();
    }
    have = logical_item(p, first, w);
  }
  if (!have) {
    if (persistent && tid == 0) sched_finish(p);
    return;
  }

  const int kv_len = p.kv_len;
  const int mkind = p.mask.kind;
  const int window = p.mask.window;
  constexpr bool doc_mask = DOC;
  const int64_t kstride = p.ks[2] * 2;  // bytes
  const int64_t vstride = p.vs[2] * 2;
  const int nkvb = p.nkvb;

  // ---- per-lane byte offsets, fixed for the whole launch
  int k_rd[DK];  // K operand: row lq (+32 jt), chunk 2dk + g
  {
    const int s = kv_swizzle<D>(lq);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) k_rd[dk] = lq * RB + (((2 * dk + g) ^ s) << 4);
  }
  int v_rd[2][DT];  // V^T operand: row 8*t2 + 4g + (lane%16)/4 (+16 kk)
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int r = 8 * t2 + 4 * g + ((lane & 15) >> 2);
    const int s = kv_swizzle<D>(r);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      v_rd[t2][dt] = r * RB + (((d >> 3) ^ s) << 4) + ((d & 7) << 1);
    }
  }
  uint32_t dma_k[ROUNDS];  // DMA: byte offset of this lane's chunk from the
  uint32_t dma_v[ROUNDS];  // stage's first K / V row
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int r = (rd * NW + wave) * RPK + lane / CPR;
    const uint32_t col = static_cast<uint32_t>(((lane % CPR) ^ kv_swizzle<D>(r)) * 16);
    dma_k[rd] = static_cast<uint32_t>(r * kstride) + col;
    dma_v[rd] = static_cast<uint32_t>(r * vstride) + col;
  }

  // ---- an item's uniform state: its key/value heads, block lists and
  // visits (split-KV part w.c of nsplit visits [v0, v0 + nvis) of the row)
  struct Item {
    WorkItem w;
    const char* kbase;
    const char* vbase;
    const int* doc;       // document ids of this batch entry
    const const_i32* pl;  // partial list, through the constant address
    const const_i32* fl;  // space: uniform scalar loads, tracked by
    int np, nf, v0, nvis; // lgkmcnt (never waits on tile DMA)
                          // stages with keys:
    int nstages;
  };
  auto make_item = [&](const WorkItem& wi0) -> Item {
    KArgs& p = kargs();
    // (uniform by construction; stated so that every derived address is
    // scalar)
    WorkItem wi;
    wi.b = __builtin_amdgcn_readfirstlane(wi0.b);
    wi.h = __builtin_amdgcn_readfirstlane(wi0.h);
    wi.m = __builtin_amdgcn_readfirstlane(wi0.m);
    wi.c = __builtin_amdgcn_readfirstlane(wi0.c);
    Item u;
    u.w = wi;
    const int hk = wi.h / (p.H / p.H_kv);
    u.kbase = reinterpret_cast<const char*>(
        static_cast<const __bf16*>(p.k) + wi.b * p.ks[0] + hk * p.ks[1]);
    u.vbase = reinterpret_cast<const char*>(
        static_cast<const __bf16*>(p.v) + wi.b * p.vs[0] + hk * p.vs[1]);
    u.doc = p.mask.doc_id + static_cast<int64_t>(wi.b) * p.mask.doc_stride;
    // the row's block lists (broadcast over batch / head when Bm / Hm is 1)
    const int bb = p.Bm == 1 ? 0 : wi.b;
    const int hh = p.Hm == 1 ? 0 : wi.h;
    const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + wi.m;
    u.nf = p.fnum ? min(max(((const const_i32*)p.fnum)[lrow], 0), nkvb) : 0;
    u.np = min(max(((const const_i32*)p.num)[lrow], 0), nkvb);
    u.fl = hw::uniform_ptr((const const_i32*)(p.fidx ? p.fidx + lrow * nkvb : p.idx));
    u.pl = hw::uniform_ptr((const const_i32*)(p.idx + lrow * nkvb));
    u.kbase = hw::uniform_ptr(u.kbase);
    u.vbase = hw::uniform_ptr(u.vbase);
    u.doc = hw::uniform_ptr(u.doc);
    const int nblocks = u.nf + u.np;
    const int per_part = (nblocks + p.nsplit - 1) / p.nsplit;
    u.v0 = min(wi.c * per_part, nblocks);
    u.nvis = min(per_part, nblocks - u.v0);
    u.nstages = u.nvis * SPB;
    return u;
  };

  // visiting order: partial blocks, then full blocks, each list from the
  // last block to the first; inside a block the later 64 keys come first
  // (`it` counts the visits of this workgroup's part)
  auto block_at = [&](const Item& u, int it) -> int {
    const int v = u.v0 + it;
    // (the list pointers restated as uniform where they are used: the
    // lookup must be a scalar load, which never waits on tile DMA)
    return v < u.np ? hw::uniform_ptr(u.pl)[u.np - 1 - v]
                    : hw::uniform_ptr(u.fl)[u.nf - 1 - (v - u.np)];
  };
  auto masked_at = [&](const Item& u, int it, int n) -> bool {
    return u.v0 + it < u.np || (n + 1) * BK > kv_len;
  };
  // block of stage st (one scalar load per key block: the stages of a block
  // share it); -1 past the item's last stage or for an index outside
  // [0, nkvb)
  auto stage_block = [&](const Item& u, int st) -> int {
    if (st >= u.nstages) return -1;
    const int b = block_at(u, st / SPB);
    return static_cast<unsigned>(b) < static_cast<unsigned>(nkvb) ? b : -1;
  };

  // Issue the DMA of stage `st` (block n) of item u into one buffer. Each
  // tile is read through a buffer resource whose base is the stage's first
  // row and whose size ends at the sequence end: rows past it read as zeros
  // (the hardware range check), so the tail needs no special path.
  auto issue = [&](const Item& u, int st, int n, char* sK, char* sV, int* sD) {
    // (uniform; stated so that the buffer descriptors are scalar)
    n = __builtin_amdgcn_readfirstlane(n);
    st = __builtin_amdgcn_readfirstlane(st);
    if (n < 0) return;
    const int it = st / SPB;
    const int j0 = n * BK + (SPB - 1 - st % SPB) * kStageKeys;
    // Rows of the stage inside the sequence. A stage of the last, ragged
    // key block may lie wholly past the end (its later keys come first):
    // then the buffers have size 0 and the tiles arrive as zeros.
    const int rows_left = kv_len - j0;
    const int krec = rows_left >= kStageKeys ? 0x7fffffff
                     : rows_left <= 0       ? 0
                                            : (rows_left - 1) * static_cast<int>(kstride) + RB;
    const int vrec = rows_left >= kStageKeys ? 0x7fffffff
                     : rows_left <= 0       ? 0
                                            : (rows_left - 1) * static_cast<int>(vstride) + RB;
    const hw::i32x4 kr = hw::make_rsrc(u.kbase + (rows_left > 0 ? j0 * kstride : 0), krec);
    const hw::i32x4 vr = hw::make_rsrc(u.vbase + (rows_left > 0 ? j0 * vstride : 0), vrec);
    // this wave's 1 KB segments: base + wave KB (+ NW KB per round)
    const uint32_t lk = hw::opaque_u32(hw::lds_addr(sK) + wave * 1024);
    const uint32_t lv = lk + static_cast<uint32_t>(sV - sK);
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      hw::dma_tile16(kr, lk + rd * NW * 1024, dma_k[rd], 0);
      hw::dma_tile16(vr, lv + rd * NW * 1024, dma_v[rd], 0);
    }
    if constexpr (doc_mask) {
      if (masked_at(u, it, n) && wave == 0) {
      const int j = min(j0 + lane, kv_len - 1);
      hw::dma_dword(u.doc, hw::lds_addr(sD), static_cast<uint32_t>(j * 4));
      }
    }
  };

  // Q^T as the MFMA B operand: column = query lq, k slots d in [16dk + 8g, +8)
  bf16x8 qf[DK];
  auto load_q = [&](const WorkItem& wi) {
    KArgs& p = kargs();
    const int i = wi.m * BQ + wave * 32 + lq;
    const bool ok = i < p.q_len;
    const __bf16* row = static_cast<const __bf16*>(p.q) + wi.b * p.qs[0] + wi.h * p.qs[1] +
                        static_cast<int64_t>(ok ? i : 0) * p.qs[2];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      u32x4 x = ok ? *reinterpret_cast<const u32x4*>(row + dk * 16 + g * 8)
                   : u32x4{0u, 0u, 0u, 0u};
      qf[dk] = __builtin_bit_cast(bf16x8, x);
    }
  };
  auto load_di = [&](const Item& u) -> int {
    const int i = u.w.m * BQ + wave * 32 + lq;
    if constexpr (doc_mask) return u.doc[i < p.q_len ? i : 0];
    return 0;
  };

  Item cur = make_item(w);
  load_q(cur.w);
  int di = load_di(cur);
  // the setup loads (Q, document id) complete before the first tile DMA, so
  // the per-stage waits below only ever wait for tiles
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  issue(cur, 0, stage_block(cur, 0), sK0, sV0, sDoc0);

  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // persistent schedule, lane 0 of wave 0 only: the counter value asked for
  // (xs: the XCD range it came from)
  unsigned pending = 0;

  for (;;) {
    // ---- this item's per-lane terms
    const int i = cur.w.m * BQ + wave * 32 + lq;
    const bool i_ok = i < kargs().q_len;
    const ScoreConsts sc = make_score_consts(kargs(), cur.w.h);
    // ALiBi: the S product starts from the key offsets of a 32-key tile in
    // units of q.k (register r of a tile holds key 8(r/4) + r%4 of the lane's
    // group), so the accumulator leaves the MFMA as q.k + jl slope / scale and
    // the bias costs no vector instruction per score
    f32x16 s_init = f32x16{};
    if constexpr (SCORE == FA_SCORE_ALIBI) {
      const float u = sc.slope2 / sc.c;  // slope / scale
#pragma unroll
      for (int r = 0; r < 16; ++r) s_init[r] = static_cast<float>(8 * (r >> 2) + (r & 3)) * u;
    }
    // mask_mod as an interval of key indices per row: j in [lo_abs, lo_abs + span)
    // (64-bit so that any window >= 1 is exact; keys are >= 0, so the
    // interval start is clamped there)
    const int hi_abs =
        mkind == FA_MASK_NONE ? kv_len
        : mkind == FA_MASK_LOCAL_WINDOW
            ? static_cast<int>(min(static_cast<int64_t>(i) + window, static_cast<int64_t>(kv_len)))
            : min(i + 1, kv_len);
    const int lo_abs =
        (mkind == FA_MASK_SLIDING_WINDOW || mkind == FA_MASK_LOCAL_WINDOW)
            ? static_cast<int>(max(static_cast<int64_t>(i) - window + 1, static_cast<int64_t>(0)))
            : 0;
    const unsigned span = static_cast<unsigned>(max(hi_abs - lo_abs, 0));

    // soft-cap with a bounded cap: fixed reference (uniform over the launch)
    const bool cap_fixed = SCORE == FA_SCORE_SOFTCAP && sc.cap_out <= kCapFixedRefMax;
    float m_run = cap_fixed ? sc.cap_out - kCapHeadroom : FA_NEG_INF;  // reference, log2 domain
    float l_run = 0.0f;        // this lane's share of the row sum, in two
    float l_run2 = 0.0f;       // independent accumulators
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

    // the next item (persistent schedule, logical index, -1 for none):
    // known to every wave from the top of stage 1 on; its first stage is
    // fetched during this item's last stage
    int next_logical = -1;
    auto compute = [&](int st, int n, const char* sK, const char* sV, const int* sD) {
      const int it = st / SPB;
      if (n < 0) return;
      const bool masked = masked_at(cur, it, n);
      const int j0 = n * BK + (SPB - 1 - st % SPB) * kStageKeys;

      // ---- S^T = K Q^T for the stage's 64 keys, at normal priority (see the
      // PV product below)
      __builtin_amdgcn_s_setprio(0);
      f32x16 s[2];
      s[0] = s_init;
      s[1] = s_init;
      u32x4 ka[DK][2];
#pragma unroll
      for (int dk = 0; dk < DK; ++dk)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          ka[dk][jt] = *reinterpret_cast<const u32x4*>(sK + k_rd[dk] + jt * 32 * RB);
#pragma unroll
      for (int dk = 0; dk < DK; ++dk)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[dk][jt]),
                                                          qf[dk], s[jt], 0, 0, 0);
      // K operand reads kept kSReadAhead ahead of the products that use them
      // (left to itself the scheduler issues each read just before its
      // product and waits on it)
      __builtin_amdgcn_sched_group_barrier(0x100, kSReadAhead, 0);  // LDS reads
#pragma unroll
      for (int t = 0; t < 2 * DK - kSReadAhead; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kSReadAhead, 0);

      // (the loads replace Q: they must not be scheduled above the S product)

      // ---- score_mod, mask_mod and the row max. Every score ends up as a
      // value x whose log2-domain score is one FMA away, s2 = x sa + sb
      // (sa, sb fixed for the lane over the stage), so the exponent below is
      // one FMA and one exp2 per score:
      //   NONE     x = q.k                        sa = scale log2e, sb = 0
      //   ALIBI    x = q.k + jl slope / scale     sa = scale log2e,
      //            (jl = the key's offset in its    sb = slope log2e (j0 + 4g - i)
      //            32-key tile; added by the S      (+ 32 slope log2e for tile 1)
      //            product through its start value)
      //   SOFTCAP  full stage: x = 1 / (e^{2 q.k scale / cap} + 1),
      //            sa = -2 cap log2e, sb = cap log2e (cap tanh = cap - 2 cap x);
      //            the row max is taken on q.k (tanh is increasing) before x is
      //            formed. Masked stage: x = s2 itself (sa = 1, sb = 0).
      // Key of (jt, r): j0 + 4g + 32jt + 8(r/4) + r%4; masked keys get x =
      // -inf before the max (p = 0).
      float sa, sb;
      bool series = false;   // soft-cap: this stage takes tanh's series,
      bool series3 = false;  // to y^3 only
      float sb1;  // (ALiBi: tile 1's offset; the other score_mods use sb for both tiles)
      float mx4[4] = {FA_NEG_INF, FA_NEG_INF, FA_NEG_INF, FA_NEG_INF};
      // max of this lane's 32 values (four independent chains); the lane
      // ^ 32 holds the row's other keys, exchanged by row_pair_max once the
      // value is in a form both lanes share
      auto lane_max = [&]() -> float {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int r = 0; r < 8; ++r) mx4[c] = __builtin_fmaxf(mx4[c], s[c >> 1][8 * (c & 1) + r]);
        return __builtin_fmaxf(__builtin_fmaxf(mx4[0], mx4[1]), __builtin_fmaxf(mx4[2], mx4[3]));
      };
      // the same, per 32-key tile
      auto lane_max2 = [&](float& m0, float& m1) {
        float t4[4] = {FA_NEG_INF, FA_NEG_INF, FA_NEG_INF, FA_NEG_INF};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int r = 0; r < 8; ++r) t4[c] = __builtin_fmaxf(t4[c], s[c >> 1][8 * (c & 1) + r]);
        m0 = __builtin_fmaxf(t4[0], t4[1]);
        m1 = __builtin_fmaxf(t4[2], t4[3]);
      };
      auto apply_mask = [&]() {
        const int lo = lo_abs - (j0 + 4 * g);  // interval start, lane-relative
        if constexpr (doc_mask) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int jl = 32 * jt + 8 * r4;
              const int4 t = *reinterpret_cast<const int4*>(sD + 4 * g + jl);
              const int dj[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const bool ok = (static_cast<unsigned>(jl + c - lo) < span) & (dj[c] == di);
                s[jt][4 * r4 + c] = ok ? s[jt][4 * r4 + c] : FA_NEG_INF;
              }
            }
        } else {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int jl = 32 * jt + 8 * (r >> 2) + (r & 3);
              s[jt][r] = static_cast<unsigned>(jl - lo) < span ? s[jt][r] : FA_NEG_INF;
            }
        }
      };
      float mx;  // row max in the log2 domain
      if constexpr (SCORE == FA_SCORE_ALIBI) {
        // x = q.k + jl slope / scale from the product; tile jt's keys start
        // 32 jt later, which its own offset sb1 carries
        sa = sc.c;
        sb = sc.slope2 * static_cast<float>(j0 + 4 * g - i);
        sb1 = __builtin_fmaf(32.0f, sc.slope2, sb);
        if (masked) apply_mask();
        // (sb differs between the two halves of the row: exchange in the
        // log2 domain; -inf stays -inf)
        float m0, m1;
        lane_max2(m0, m1);
        mx = row_pair_max(__builtin_fmaxf(__builtin_fmaf(m0, sa, sb), __builtin_fmaf(m1, sa, sb1)));
      } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
        const float k2 = 2.0f * sc.cap_in * kLog2e;
        mx = FA_NEG_INF;  // (fixed reference: no maximum)
        bool small = false, small3 = false;
        if (cap_fixed) {
          // the series when every score of the wave's stage is small enough
          // (uniform; a NaN score gives a NaN weight on either path)
          float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 8; ++r)
              a4[c] = __builtin_fmaxf(a4[c], __builtin_fabsf(s[c >> 1][8 * (c & 1) + r]));
          const float amax = __builtin_fmaxf(__builtin_fmaxf(a4[0], a4[1]), __builtin_fmaxf(a4[2], a4[3]));
          small = __builtin_amdgcn_ballot_w64(!(amax * sc.cap_in <= kCapSeriesY)) == 0;
          small3 = small &&
                   __builtin_amdgcn_ballot_w64(!(amax * sc.cap_in <= kCapSeries3Y)) == 0;
        }
        series = small && !masked;
        series3 = small3 && !masked;
        if (series) {
          sa = 0.0f;  // (the series path forms its own multiplier per score)
          sb = 0.0f;
        } else if (!masked) {
          if (!cap_fixed) {
            const float mraw = row_pair_max(lane_max());
            mx = mraw == FA_NEG_INF
                     ? FA_NEG_INF
                     : __builtin_fmaf(-2.0f * sc.cap_out,
                                      __builtin_amdgcn_rcpf(exp2_hw(mraw * k2) + 1.0f),
                                      sc.cap_out);
          }
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[jt][r] = __builtin_amdgcn_rcpf(exp2_hw(s[jt][r] * k2) + 1.0f);
          sa = -2.0f * sc.cap_out;
          sb = sc.cap_out;
        } else {
          // masked stage: the capped score itself (log2 domain), then the mask
          if (small) {
            // (the series as below, on the capped score rather than in the exponent)
            const float a = sc.cap_in, a2 = a * a;
            const float c0 = sc.cap_out * a, c1 = -c0 * a2 * (1.0f / 3.0f),
                        c2 = c0 * a2 * a2 * (2.0f / 15.0f);
            if (small3) {
#pragma unroll
              for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float x = s[jt][r];
                  s[jt][r] = x * __builtin_fmaf(x * x, c1, c0);
                }
            } else {
#pragma unroll
              for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float x = s[jt][r], t = x * x;
                  s[jt][r] = x * __builtin_fmaf(t, __builtin_fmaf(t, c2, c1), c0);
                }
            }
          } else {
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float t = __builtin_amdgcn_rcpf(exp2_hw(s[jt][r] * k2) + 1.0f);
                s[jt][r] = __builtin_fmaf(-2.0f * sc.cap_out, t, sc.cap_out);
              }
          }
          apply_mask();
          if (!cap_fixed) mx = row_pair_max(lane_max());
          sa = 1.0f;
          sb = 0.0f;
        }
      } else {
        if (masked) apply_mask();
        mx = row_pair_max(lane_max()) * sc.c;  // raw -> log2 domain
        sa = sc.c;
        sb = 0.0f;
      }

      // ---- online softmax: lazy rescale, then p = exp2(s2 - m_ref)
      const bool raise = mx > m_run + kRescaleSlack;
      if (!cap_fixed && __builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = (m_new == m_run) ? 1.0f : exp2_hw(m_run - m_new);
        l_run *= alpha;
        l_run2 *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == FA_NEG_INF) ? 0.0f : m_run;
      if constexpr (SCORE != FA_SCORE_ALIBI) sb1 = sb;
      const float ofs[2] = {sb - m_use, sb1 - m_use};
      bf16x8 pb[4];
      // p = exp2(x mul(x) + ofs): mul is sa, or on a series stage the odd
      // series' polynomial in x^2, so that s2 = x (c0 + x^2 (c1 + x^2 c2))
      auto weights = [&](auto mul_of) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          f32x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[kk >> 1][(kk & 1) * 8 + e];
            pf[e] = exp2_hw(__builtin_fmaf(x, mul_of(x), ofs[kk >> 1]));
          }
          pb[kk] = __builtin_convertvector(pf, bf16x8);
          const u32x4 pw = __builtin_bit_cast(u32x4, pb[kk]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // copy the word out first: bit-casting a vector element in place
            // mis-compiles (every iteration reads element 0)
            const uint32_t word = pw[e];
            float& acc = (e & 1) ? l_run2 : l_run;
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), ones, acc,
                                                  false);
          }
        }
      };
      if (SCORE == FA_SCORE_SOFTCAP && series) {
        // cap tanh(a x) log2 e = x (c0 + x^2 (c1 + x^2 c2)), a = scale / cap
        const float a = sc.cap_in, a2 = a * a;
        const float c0 = sc.cap_out * a;
        const float c1 = -c0 * a2 * (1.0f / 3.0f);
        const float c2 = c0 * a2 * a2 * (2.0f / 15.0f);
        if (series3) {
          weights([&](float x) { return __builtin_fmaf(x * x, c1, c0); });
        } else {
          weights([&](float x) {
            const float t = x * x;
            return __builtin_fmaf(t, __builtin_fmaf(t, c2, c1), c0);
          });
        }
      } else {
        weights([&](float) { return sa; });
      }

      // ---- O^T += V^T P^T (4 k-steps of 16 keys). The wave raises its issue
      // priority from here until its next stage's S product: of the two waves
      // sharing a SIMD, the one whose P is ready gets its products issued ahead
      // of the other's softmax arithmetic, which keeps the matrix core fed.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const i16x4 lo = lds_read_tr(sV + v_rd[0][dt] + kk * 16 * RB);
          const i16x4 hi = lds_read_tr(sV + v_rd[1][dt] + kk * 16 * RB);
          const i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[kk],
                                                             oacc[dt], 0, 0, 0);
        }
      }
    };

    // ---- main loop over stages, unrolled by two so each LDS buffer is its
    // own object; the DMA of stage st + 1 overlaps the compute of stage st.
    // At the top of each stage this lane's DMA has landed (vmcnt), then
    // every lane's (barrier), which also frees the other buffer. Persistent
    // schedule: lane 0 asks for the next item after the barrier of stage 0
    // and publishes it before the barrier of stage 1; an item with an even
    // number of stages ends in buffer 1, and the next item's first stage
    // goes to buffer 0 during its last stage. n_cur: block of stage st;
    // n_nxt: of stage st + 1.
    int n_cur = stage_block(cur, 0);
    const int nstages = cur.nstages;
    bool first_issued = false;  // the next item's first stage is in flight
    for (int st = 0; st < nstages; st += 2) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (persistent && st == 0 && tid == 0)
        pending = __hip_atomic_fetch_add(kargs().sched + (xs & 7), 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      int n_nxt = st + 1 >= nstages ? -1 : (st + 1) % SPB == 0 ? stage_block(cur, st + 1) : n_cur;
      if (st + 1 < nstages) issue(cur, st + 1, n_nxt, sK1, sV1, sDoc1);
      compute(st, n_cur, sK0, sV0, sDoc0);
      if (st + 1 >= nstages) break;
      n_cur = n_nxt;
      __builtin_amdgcn_s_waitcnt(0x0f70);
      // (one counter only here; moving on to other ranges, which takes
      // further atomics, waits for the end of the item)
      if (persistent && st == 0 && tid == 0) sNext = sched_check(kargs(), pending, xs);
      __syncthreads();
      if (persistent && st == 0) next_logical = __builtin_amdgcn_readfirstlane(sNext);
      n_nxt = st + 2 >= nstages ? -1 : (st + 2) % SPB == 0 ? stage_block(cur, st + 2) : n_cur;
      if (st + 2 < nstages) {
        issue(cur, st + 2, n_nxt, sK0, sV0, sDoc0);
      } else if (next_logical >= 0) {  // (-2: not known yet)
        WorkItem wn;
        logical_item(kargs(), next_logical, wn);
        const Item u = make_item(wn);
        issue(u, 0, stage_block(u, 0), sK0, sV0, sDoc0);
        first_issued = true;
      }
      compute(st + 1, n_cur, sK1, sV1, sDoc1);
      n_cur = n_nxt;
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
    {
    KArgs& p = kargs();
    const float l_tot = row_pair_sum(l_run + l_run2);
    if (p.nsplit > 1) {
      // split-KV part: the unnormalised accumulator and (m, l) for the merge
      if (i_ok) {
        const int64_t prow =
            (static_cast<int64_t>(cur.w.c) * p.B * p.H + static_cast<int64_t>(cur.w.b) * p.H +
             cur.w.h) * p.q_len + i;
        float* po = p.part_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(po + dt * 32 + 8 * q4 + 4 * g) =
                f32x4{oacc[dt][4 * q4 + 0], oacc[dt][4 * q4 + 1], oacc[dt][4 * q4 + 2],
                      oacc[dt][4 * q4 + 3]};
        if (g == 0) {
          p.part_ml[2 * prow] = m_run;
          p.part_ml[2 * prow + 1] = l_tot;
        }
      }
    } else if (i_ok) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const int64_t orow = (static_cast<int64_t>(cur.w.b) * p.H + cur.w.h) * p.q_len + i;
      __bf16* op = static_cast<__bf16*>(p.o) + orow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v4 = {oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv,
                            oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv};
          *reinterpret_cast<bf16x4*>(op + dt * 32 + 8 * q4 + 4 * g) =
              __builtin_convertvector(v4, bf16x4);
        }
      if (g == 0 && p.lse)
        p.lse[orow] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : FA_NEG_INF;
    }
    }
    if (persistent && (nstages < 2 || next_logical == -2)) {
      // the next item was not published in the loop (fewer than two
      // stages), or this workgroup's range is used up: ask the counters,
      // moving on to the following XCDs' ranges
      if (tid == 0) {
        if (nstages == 0)
          pending = __hip_atomic_fetch_add(kargs().sched + (xs & 7), 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        if (nstages >= 2) {  // the published value was this range's last word
          if (++xs < static_cast<int>(blockIdx.x & 7) + 8)
            sNext = sched_resolve(kargs(),
                                  __hip_atomic_fetch_add(kargs().sched + (xs & 7), 1u,
                                                         __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT),
                                  xs);
          else
            sNext = -1;
        } else {
          sNext = sched_resolve(kargs(), pending, xs);
        }
      }
      __syncthreads();
      next_logical = __builtin_amdgcn_readfirstlane(sNext);
    }
    if (next_logical < 0) break;
    WorkItem wn;
    logical_item(kargs(), next_logical, wn);
    cur = make_item(wn);
    if (!first_issued) {
      // odd stage count or none: both buffers may still be read until every
      // wave is here
      __syncthreads();
      issue(cur, 0, stage_block(cur, 0), sK0, sV0, sDoc0);
    }
    // the next item's Q (its first stage is already in flight)
    load_q(cur.w);
    di = load_di(cur);
  }
  if (persistent && tid == 0) sched_finish(p);
}

}  // namespace fa
