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
// ones), i.e. exactly the weights the PV product uses.
#pragma once

#include "fwd_asm.hpp"
#include "fwd_common.hpp"

namespace fa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlack = 8.0f;
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

// Workgroup -> (head, query block, split part). Workgroups are dispatched
// round-robin over the 8 XCDs (wg % 8). Logical items are dealt to XCDs in
// contiguous ranges so that the query blocks of one head run on one XCD and
// share its L2; within a head the heaviest query blocks (last rows under
// causal masks) come first.
__device__ __forceinline__ bool xcd_work_item(const FwdLaunch& p, WorkItem& w) {
  const int total = p.B * p.H * p.nqb * p.nsplit;
  const int per_xcd = (total + 7) >> 3;
  const int wg = blockIdx.x;
  const int logical = (wg & 7) * per_xcd + (wg >> 3);
  if (logical >= total) return false;
  w.c = logical % p.nsplit;  // the parts of one query block run side by side
  const int row = logical / p.nsplit;
  w.m = p.nqb - 1 - (row % p.nqb);
  const int bh = row / p.nqb;
  w.h = bh % p.H;
  w.b = bh / p.H;
  return true;
}

template <int D, int BQ, int BK, int SCORE>
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

  __shared__ __attribute__((aligned(1024))) char sK0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int sDoc0[kStageKeys];
  __shared__ __attribute__((aligned(16))) int sDoc1[kStageKeys];

  WorkItem w;
  if (!xcd_work_item(p, w)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  const int hk = w.h / (p.H / p.H_kv);
  const int i = w.m * BQ + wave * 32 + lq;
  const bool i_ok = i < p.q_len;
  const int kv_len = p.kv_len;
  const int mkind = p.mask.kind;
  const int window = p.mask.window;
  // document ids of this batch entry (one shared array when the stride is 0)
  const int* doc = p.mask.doc_id + static_cast<int64_t>(w.b) * p.mask.doc_stride;
  const bool doc_mask = mkind == FA_MASK_DOCUMENT;

  const __bf16* qp = static_cast<const __bf16*>(p.q) + w.b * p.qs[0] + w.h * p.qs[1];
  const char* kbase = reinterpret_cast<const char*>(
      static_cast<const __bf16*>(p.k) + w.b * p.ks[0] + hk * p.ks[1]);
  const char* vbase = reinterpret_cast<const char*>(
      static_cast<const __bf16*>(p.v) + w.b * p.vs[0] + hk * p.vs[1]);
  const int64_t kstride = p.ks[2] * 2;  // bytes
  const int64_t vstride = p.vs[2] * 2;

  // Q^T as the MFMA B operand: column = query lq, k slots d in [16dk + 8g, +8)
  bf16x8 qf[DK];
  {
    const __bf16* row = qp + static_cast<int64_t>(i_ok ? i : 0) * p.qs[2];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      u32x4 x = i_ok ? *reinterpret_cast<const u32x4*>(row + dk * 16 + g * 8)
                     : u32x4{0u, 0u, 0u, 0u};
      qf[dk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const int di = doc_mask ? doc[i_ok ? i : 0] : 0;

  // the row's block lists (broadcast over batch / head when Bm / Hm is 1)
  const int bb = p.Bm == 1 ? 0 : w.b;
  const int hh = p.Hm == 1 ? 0 : w.h;
  const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + w.m;
  const int nkvb = p.nkvb;
  const int nf = p.fnum ? min(max(p.fnum[lrow], 0), nkvb) : 0;
  const int np = min(max(p.num[lrow], 0), nkvb);
  // block lists through the constant address space: uniform scalar loads,
  // tracked by lgkmcnt, so reading them never waits on in-flight tile DMA
  const const_i32* fl = (const const_i32*)(p.fidx ? p.fidx + lrow * nkvb : p.idx);
  const const_i32* pl = (const const_i32*)(p.idx + lrow * nkvb);
  const int nblocks = nf + np;
  // split-KV part w.c of nsplit: visits [v0, v0 + nvis) of the row's order
  const int per_part = (nblocks + p.nsplit - 1) / p.nsplit;
  const int v0 = min(w.c * per_part, nblocks);
  const int nvis = min(per_part, nblocks - v0);
  const int nstages = nvis * SPB;

  const ScoreConsts sc = make_score_consts(p, w.h);
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

  // ---- per-lane byte offsets, fixed for the whole row
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

  // visiting order: partial blocks, then full blocks, each list from the
  // last block to the first; inside a block the later 64 keys come first
  // (`it` counts the visits of this workgroup's part)
  auto block_at = [&](int it) -> int {
    const int v = v0 + it;
    return v < np ? pl[np - 1 - v] : fl[nf - 1 - (v - np)];
  };
  auto masked_at = [&](int it, int n) -> bool {
    return v0 + it < np || (n + 1) * BK > kv_len;
  };

  // Issue the DMA of stage `st` (block visit st / SPB) into one buffer. Each
  // tile is read through a buffer resource whose base is the stage's first
  // row and whose size ends at the sequence end: rows past it read as zeros
  // (the hardware range check), so the tail needs no special path.
  // block of stage st (one scalar load per key block: the stages of a block
  // share it), -1 for an index outside [0, nkvb)
  auto stage_block = [&](int st) -> int {
    const int b = block_at(st / SPB);
    return static_cast<unsigned>(b) < static_cast<unsigned>(nkvb) ? b : -1;
  };
  auto issue = [&](int st, int n, char* sK, char* sV, int* sD) {
    const int it = st / SPB;
    if (n < 0) return;
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
    const hw::i32x4 kr = hw::make_rsrc(kbase + (rows_left > 0 ? j0 * kstride : 0), krec);
    const hw::i32x4 vr = hw::make_rsrc(vbase + (rows_left > 0 ? j0 * vstride : 0), vrec);
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int seg = (rd * NW + wave) * 1024;
      hw::dma_tile16(kr, hw::lds_addr(sK + seg), dma_k[rd], 0);
      hw::dma_tile16(vr, hw::lds_addr(sV + seg), dma_v[rd], 0);
    }
    if (doc_mask && masked_at(it, n) && wave == 0) {
      const int j = min(j0 + lane, kv_len - 1);
      hw::dma_dword(doc, hw::lds_addr(sD), static_cast<uint32_t>(j * 4));
    }
  };

  float m_run = FA_NEG_INF;  // reference max, log2 domain
  float l_run = 0.0f;        // this lane's share of the row sum, in two
  float l_run2 = 0.0f;       // independent accumulators
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  auto compute = [&](int st, int n, const char* sK, const char* sV, const int* sD) {
    const int it = st / SPB;
    if (n < 0) return;
    const bool masked = masked_at(it, n);
    const int j0 = n * BK + (SPB - 1 - st % SPB) * kStageKeys;

    // ---- S^T = K Q^T for the stage's 64 keys, at normal priority (see the
    // PV product below)
    __builtin_amdgcn_s_setprio(0);
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
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

    // ---- score_mod into the log2 domain (NONE keeps raw q.k: c > 0 is
    // applied in the exponent). Key of (jt, r): j0 + 4g + 32jt + 8(r/4) + r%4.
    if constexpr (SCORE == FA_SCORE_ALIBI) {
      const float bias0 = sc.slope2 * static_cast<float>(j0 + 4 * g - i);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float b = __builtin_fmaf(sc.slope2, static_cast<float>(32 * jt + 8 * (r >> 2) + (r & 3)), bias0);
          s[jt][r] = __builtin_fmaf(s[jt][r], sc.c, b);
        }
    } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
      // cap * tanh(x) * log2e with tanh x = 1 - 2 / (e^{2x} + 1)
      const float k2 = 2.0f * sc.cap_in * kLog2e;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_hw(s[jt][r] * k2);
          const float t = __builtin_amdgcn_rcpf(e + 1.0f);
          s[jt][r] = __builtin_fmaf(-2.0f * sc.cap_out, t, sc.cap_out);
        }
    }

    // ---- mask_mod on partial and sequence-tail blocks only. Every built-in
    // mask bounds a row's keys to an interval (causal: j <= i, sliding
    // window: i - W < j <= i, local window: |i - j| < W, and j < kv_len),
    // so the test is one unsigned
    // compare of the key's offset in the interval against its length, plus
    // the document-id equality for document masks.
    if (masked) {
      const int lo = lo_abs - (j0 + 4 * g);  // interval start, lane-relative
      if (doc_mask) {
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
    }

    // ---- online softmax. Row max: four independent chains, then the
    // exchange with lane ^ 32 (the other half of the row's keys).
    float mx4[4] = {FA_NEG_INF, FA_NEG_INF, FA_NEG_INF, FA_NEG_INF};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) mx4[c] = __builtin_fmaxf(mx4[c], s[c >> 1][8 * (c & 1) + r]);
    float mx = __builtin_fmaxf(__builtin_fmaxf(mx4[0], mx4[1]), __builtin_fmaxf(mx4[2], mx4[3]));
    mx = row_pair_max(mx);
    if constexpr (SCORE == FA_SCORE_NONE) mx *= sc.c;  // raw -> log2 domain
    const bool raise = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_run;
      const float alpha = (m_new == m_run) ? 1.0f : exp2_hw(m_run - m_new);
      l_run *= alpha;
      l_run2 *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == FA_NEG_INF) ? 0.0f : m_run;
    bf16x8 pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = s[kk >> 1][(kk & 1) * 8 + e];
        if constexpr (SCORE == FA_SCORE_NONE) {
          pf[e] = exp2_hw(__builtin_fmaf(x, sc.c, -m_use));
        } else {
          pf[e] = exp2_hw(x - m_use);
        }
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
  // The setup loads (Q, document id) complete before the first tile DMA, so
  // the per-stage waits below only ever wait for tiles.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  // n_cur: block of stage st; n_nxt: of stage st + 1 (loaded with its DMA)
  int n_cur = nstages > 0 ? stage_block(0) : -1;
  if (nstages > 0) issue(0, n_cur, sK0, sV0, sDoc0);
  for (int st = 0; st < nstages; st += 2) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this lane's DMA landed
    __syncthreads();                     // every lane's DMA landed; buffer 1 free
    // (no lookup past the last stage: the list index would leave the row)
    int n_nxt = st + 1 >= nstages ? -1 : (st + 1) % SPB == 0 ? stage_block(st + 1) : n_cur;
    if (st + 1 < nstages) issue(st + 1, n_nxt, sK1, sV1, sDoc1);
    compute(st, n_cur, sK0, sV0, sDoc0);
    if (st + 1 >= nstages) break;
    n_cur = n_nxt;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    n_nxt = st + 2 >= nstages ? -1 : (st + 2) % SPB == 0 ? stage_block(st + 2) : n_cur;
    if (st + 2 < nstages) issue(st + 2, n_nxt, sK0, sV0, sDoc0);
    compute(st + 1, n_cur, sK1, sV1, sDoc1);
    n_cur = n_nxt;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = row_pair_sum(l_run + l_run2);
  if (p.nsplit > 1) {
    // split-KV part: the unnormalised accumulator and (m, l) for the merge
    if (i_ok) {
      const int64_t prow =
          (static_cast<int64_t>(w.c) * p.B * p.H + static_cast<int64_t>(w.b) * p.H + w.h) *
              p.q_len + i;
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
    return;
  }
  if (i_ok) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t orow = (static_cast<int64_t>(w.b) * p.H + w.h) * p.q_len + i;
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

}  // namespace fa
