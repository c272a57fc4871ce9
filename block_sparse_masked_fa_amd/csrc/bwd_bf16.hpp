// Backward of the fused block-sparse attention, bf16 inputs and gradients,
// fp32 accumulation, for gfx950. Gradients of O = attention(Q, K, V) for an
// upstream dO (the LSE output is not differentiated), over the same block
// mask as the forward, by the chain rule through the masked softmax and the
// score_mod:
//
//   t = scale q.k,  s = score_mod(t),  P_ij = exp(s_ij - LSE_i) (allowed),
//   dV_j = sum_i P_ij dO_i,       dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - delta_i) with delta_i = dO_i . O_i,
//   dT = dS * score_mod'(t)  (1 for none / ALiBi, 1 - tanh^2 for soft-cap),
//   dQ_i = scale sum_j dT_ij k_j,  dK_j = scale sum_i dT_ij q_i.
//
// The forward's LSE makes P available per tile with no running maximum, so
// every tile is independent and two kernels avoid atomics:
//   * bwd_dq_kernel: one workgroup per (query block, head), the forward's
//     work split and key-block lists. It first forms delta_i from its rows
//     of O and dO (and stores it for the next kernel). Per 64-key stage:
//     S^T = K Q^T and dP^T = V dO^T (K and V rows as MFMA A operands from
//     LDS, Q^T and dO^T resident as B operands), then dQ^T += K^T dT^T (K
//     read transposed, ds_read_b64_tr_b16, exactly as the forward reads V).
//   * bwd_dkdv_kernel: one workgroup per (key block, key head), wave w owns
//     keys [32w, 32w + 32); it walks the transposed lists (the query blocks
//     that name the key block) and, with grouped heads, every query head of
//     the group. Per 64-row stage of Q and dO in LDS (with each row's
//     delta and exponent offset, which the dQ kernel stores): S = Q K^T and
//     dP = dO V^T (K^T and V^T resident as B operands), then
//     dV^T += dO^T P and dK^T += Q^T dT (dO and Q read transposed).
// The layouts, swizzles and loads are the forward's (fwd_bf16.hpp). With
// the roles of queries and keys exchanged in bwd_dkdv_kernel, a lane's
// accumulator values share one key and span 16 query rows, so the per-row
// terms (exponent offset, delta, document id) come from LDS and mask_mod is
// an interval of query rows per key.
#pragma once

#include <type_traits>

#include "fwd_bf16.hpp"

namespace fa {

// A per-lane value the compiler cannot see through: formed where it is used
// instead of being folded into other expressions or held across a loop.
__device__ __forceinline__ int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The soft-cap's derivative enters dT as t (1 - t) with t = 1 / (e^{2x} + 1),
// which is (1 - tanh^2 x) / 4; the factor 4, a power of two, is applied to
// the fp32 sums at the end (exact: scaling by 4 commutes with rounding).
constexpr float kSoftcapGrad = 4.0f;

// Workgroup -> (batch, key head, key block) for the dK / dV kernel: dealt to
// the 8 XCDs in contiguous ranges (one head's blocks share an L2).
template <class Params>
__device__ __forceinline__ bool xcd_kv_item(const Params& p, int nsplit, int& b, int& hk, int& n,
                                            int& c) {
  const int total = p.B * p.H_kv * p.nkvb * nsplit;
  const int per_xcd = (total + 7) >> 3;
  const int wg = blockIdx.x;
  const int logical = (wg & 7) * per_xcd + (wg >> 3);
  if (logical >= total) return false;
  c = logical % nsplit;  // the parts of one key block run side by side
  const int item = logical / nsplit;
  n = item % p.nkvb;
  const int bh = item / p.nkvb;
  hk = bh % p.H_kv;
  b = bh / p.H_kv;
  return true;
}

// ---------------------------------------------------------------- dQ
template <int D, int BQ, int BK, int SCORE>
__global__ __launch_bounds__(BQ * 2, 256 / BQ) void bwd_dq_kernel(const BwdLaunch bp) {
  const FwdLaunch& p = bp.f;
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  constexpr int SPB = BK / kStageKeys;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPK = 1024 / RB;
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
  const int* doc = p.mask.doc_id + static_cast<int64_t>(w.b) * p.mask.doc_stride;
  const bool doc_mask = mkind == FA_MASK_DOCUMENT;

  const __bf16* qp = static_cast<const __bf16*>(p.q) + w.b * p.qs[0] + w.h * p.qs[1];
  const int64_t orow = (static_cast<int64_t>(w.b) * p.H + w.h) * p.q_len + i;
  const __bf16* dop = static_cast<const __bf16*>(bp.dout) + (i_ok ? orow : 0) * D;
  const char* kbase = reinterpret_cast<const char*>(
      static_cast<const __bf16*>(p.k) + w.b * p.ks[0] + hk * p.ks[1]);
  const char* vbase = reinterpret_cast<const char*>(
      static_cast<const __bf16*>(p.v) + w.b * p.vs[0] + hk * p.vs[1]);
  const int64_t kstride = p.ks[2] * 2;
  const int64_t vstride = p.vs[2] * 2;

  // Q^T and dO^T as MFMA B operands: column = query lq, k slots d in
  // [16dk + 8g, +8)
  bf16x8 qf[DK], dof[DK];
  {
    const __bf16* row = qp + static_cast<int64_t>(i_ok ? i : 0) * p.qs[2];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[dk] = __builtin_bit_cast(bf16x8, i_ok ? *reinterpret_cast<const u32x4*>(row + dk * 16 + g * 8) : z);
      dof[dk] = __builtin_bit_cast(bf16x8, i_ok ? *reinterpret_cast<const u32x4*>(dop + dk * 16 + g * 8) : z);
    }
  }
  // log2-domain LSE (a row without keys: +inf, so that every P is 0)
  const float lse_i = i_ok ? bp.lse[orow] : FA_NEG_INF;
  const float lse2 = lse_i == FA_NEG_INF ? __builtin_inff() : lse_i * kLog2e;
  // delta_i = dO_i . O_i (fp32), the row term of dS; written for the dK / dV
  // kernel, which runs after this one. Each lane holds the row's d in
  // [16 dk + 8 g, +8): a partial dot, then the sum with lane ^ 32.
  float delta_i;
  {
    const __bf16* orow_p = static_cast<const __bf16*>(bp.o) + (i_ok ? orow : 0) * D;
    float part = 0.0f;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const bf16x8 ov = __builtin_bit_cast(
          bf16x8, i_ok ? *reinterpret_cast<const u32x4*>(orow_p + dk * 16 + g * 8) : z);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        part = __builtin_fmaf(static_cast<float>(ov[e]), static_cast<float>(dof[dk][e]), part);
    }
    delta_i = row_pair_sum(part);
    if (i_ok && g == 0 && w.c == 0) {
      bp.delta[orow] = delta_i;
      // the row's exponent offset for the dK / dV kernel
      float rt = lse_i == FA_NEG_INF ? FA_NEG_INF : -lse_i * kLog2e;
      if (SCORE == FA_SCORE_ALIBI && lse_i != FA_NEG_INF)
        rt -= make_score_consts(p, w.h).slope2 * static_cast<float>(i);
      bp.rowterm[orow] = rt;
    }
  }
  const int di = doc_mask ? doc[i_ok ? i : 0] : 0;

  const int bb = p.Bm == 1 ? 0 : w.b;
  const int hh = p.Hm == 1 ? 0 : w.h;
  const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + w.m;
  const int nkvb = p.nkvb;
  const int nf = p.fnum ? min(max(p.fnum[lrow], 0), nkvb) : 0;
  const int np = min(max(p.num[lrow], 0), nkvb);
  const const_i32* fl = (const const_i32*)(p.fidx ? p.fidx + lrow * nkvb : p.idx);
  const const_i32* pl = (const const_i32*)(p.idx + lrow * nkvb);
  const int nblocks = nf + np;
  // part w.c of p.nsplit: block visits [v0, v0 + nvis) of the merged order
  const int per_part = (nblocks + p.nsplit - 1) / p.nsplit;
  const int v0 = min(w.c * per_part, nblocks);
  const int nvis = min(per_part, nblocks - v0);
  const int nstages = nvis * SPB;

  const ScoreConsts sc = make_score_consts(p, w.h);
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

  // per-lane LDS offsets, as in the forward: rows as A operands and the
  // transposed reads
  int k_rd[DK];
  {
    const int s = kv_swizzle<D>(lq);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) k_rd[dk] = lq * RB + (((2 * dk + g) ^ s) << 4);
  }
  int v_rd[2][DT];
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
  uint32_t dma_k[ROUNDS], dma_v[ROUNDS];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int r = (rd * NW + wave) * RPK + lane / CPR;
    const uint32_t col = static_cast<uint32_t>(((lane % CPR) ^ kv_swizzle<D>(r)) * 16);
    dma_k[rd] = static_cast<uint32_t>(r * kstride) + col;
    dma_v[rd] = static_cast<uint32_t>(r * vstride) + col;
  }

  // dQ accumulation order: the row's live key blocks, the partial and the
  // full list merged by block index, in ascending (dq_kv_order 0) or
  // descending (1) order; descending also takes a block's later 64 keys
  // first. Each list is walked in its own order, which the builder sorts.
  // Fixed for given inputs, so dQ is bitwise reproducible.
  const bool desc = bp.dq_kv_order != 0;
  int ip = desc ? np - 1 : 0;
  int ifl = desc ? nf - 1 : 0;
  int c_n = -1, c_sub = 0;
  bool c_masked = false;
  // this part's first visit: skip v0 blocks of the merged order
  for (int v = 0; v < v0; ++v) {
    const bool p_left = desc ? ip >= 0 : ip < np;
    const bool f_left = desc ? ifl >= 0 : ifl < nf;
    bool take_p = p_left;
    if (p_left && f_left) take_p = desc ? pl[ip] > fl[ifl] : pl[ip] < fl[ifl];
    if (take_p) ip += desc ? -1 : 1;
    else ifl += desc ? -1 : 1;
  }
  // the next stage: key block n (-1: an index outside [0, NKVB), skipped),
  // its 64-key stage sub, and whether mask_mod applies. Called once per
  // stage, in order, nstages times.
  auto next_stage = [&](int& n, int& sub, bool& masked) {
    if (c_sub == 0) {
      const bool p_left = desc ? ip >= 0 : ip < np;
      const bool f_left = desc ? ifl >= 0 : ifl < nf;
      bool take_p = p_left;
      if (p_left && f_left) {
        const int a = pl[ip], bq = fl[ifl];
        take_p = desc ? a > bq : a < bq;
      }
      const int bsel = take_p ? pl[ip] : fl[ifl];
      if (take_p) ip += desc ? -1 : 1;
      else ifl += desc ? -1 : 1;
      c_n = static_cast<unsigned>(bsel) < static_cast<unsigned>(nkvb) ? bsel : -1;
      c_masked = take_p || (c_n + 1) * BK > kv_len;
    }
    n = c_n;
    sub = desc ? SPB - 1 - c_sub : c_sub;
    masked = c_masked;
    if (++c_sub == SPB) c_sub = 0;
  };
  auto issue = [&](int n, int sub, bool masked, char* sK, char* sV, int* sD) {
    if (n < 0) return;
    const int j0 = n * BK + sub * kStageKeys;
    // a stage of a ragged last block may lie wholly past the end: then the
    // buffers have size 0 and the tiles arrive as zeros
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
    if (doc_mask && masked && wave == 0) {
      const int j = min(j0 + lane, kv_len - 1);
      hw::dma_dword(doc, hw::lds_addr(sD), static_cast<uint32_t>(j * 4));
    }
  };

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  auto compute = [&](int n, int sub, bool masked, const char* sK, const char* sV,
                     const int* sD) {
    if (n < 0) return;
    const int j0 = n * BK + sub * kStageKeys;

    // Two halves of 32 keys each (jt), one after the other (one S and one
    // dP tile live at a time); each half's LDS operands are read ahead of
    // its MFMAs.
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      // S^T = K Q^T and dP^T = V dO^T for keys [32 jt, 32 jt + 32)
      f32x16 s = f32x16{}, dp = f32x16{};
      u32x4 ka[DK], va[DK];
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        ka[dk] = *reinterpret_cast<const u32x4*>(sK + k_rd[dk] + jt * 32 * RB);
        va[dk] = *reinterpret_cast<const u32x4*>(sV + k_rd[dk] + jt * 32 * RB);
      }
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[dk]), qf[dk], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[dk]), dof[dk],
                                                     dp, 0, 0, 0);
      }

      // P = 2^(score_mod in the log2 domain - LSE log2 e), with the row's
      // LSE folded into the exponent's FMA, and score_mod' (soft-cap); key of
      // element r: j0 + 32 jt + 8 (r / 4) + 4 g + r % 4. A row without keys
      // has lse2 = +inf: every P is 0.
      float fp[16];
      // ALiBi bias slope2 (j - i) = bias0 + slope2 (8 (r / 4) + r % 4)
      const float bias0 =
          SCORE == FA_SCORE_ALIBI
              ? sc.slope2 * static_cast<float>(j0 + 4 * g + 32 * jt - i) - lse2
              : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        fp[r] = 1.0f;
        float arg;
        if constexpr (SCORE == FA_SCORE_ALIBI) {
          const float bj =
              __builtin_fmaf(sc.slope2, static_cast<float>(8 * (r >> 2) + (r & 3)), bias0);
          arg = __builtin_fmaf(s[r], sc.c, bj);
        } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
          const float e = exp2_hw(s[r] * (2.0f * sc.cap_in * kLog2e));
          const float tt = __builtin_amdgcn_rcpf(e + 1.0f);  // tanh = 1 - 2 tt
          arg = __builtin_fmaf(-2.0f * sc.cap_out, tt, sc.cap_out - lse2);
          fp[r] = __builtin_fmaf(-tt, tt, tt);  // (1 - tanh^2) / 4
        } else {
          arg = __builtin_fmaf(s[r], sc.c, -lse2);
        }
        s[r] = exp2_hw(arg);
      }
      // mask_mod on partial and tail stages only (a uniform branch)
      if (masked) {
        const int lo = lo_abs - (j0 + 4 * g);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int jl = 32 * jt + 8 * r4;
          int dj[4] = {di, di, di, di};
          if (doc_mask) {
            const int4 t = *reinterpret_cast<const int4*>(sD + 4 * g + jl);
            dj[0] = t.x; dj[1] = t.y; dj[2] = t.z; dj[3] = t.w;
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool ok = (static_cast<unsigned>(jl + c - lo) < span) & (dj[c] == di);
            s[4 * r4 + c] = ok ? s[4 * r4 + c] : 0.0f;
          }
        }
      }

      // dS = P (dP - delta), dT = dS score_mod' -> bf16 B operands
      bf16x8 tb[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x8 tf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = h2 * 8 + e;
          tf[e] = s[r] * (dp[r] - delta_i) * fp[r];
        }
        tb[h2] = __builtin_convertvector(tf, bf16x8);
      }

      // dQ^T += K^T dT^T over these 32 keys (2 k-steps of 16; K read
      // transposed)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int kk = 2 * jt + h2;
        i16x8 a8[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const i16x4 lo = lds_read_tr(sK + v_rd[0][dt] + kk * 16 * RB);
          const i16x4 hi = lds_read_tr(sK + v_rd[1][dt] + kk * 16 * RB);
          a8[dt] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8[dt]),
                                                           tb[h2], dq[dt], 0, 0, 0);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): setup loads landed
  int n_cur = -1, sub_cur = 0, n_nxt = -1, sub_nxt = 0;
  bool mk_cur = false, mk_nxt = false;
  if (nstages > 0) {
    next_stage(n_cur, sub_cur, mk_cur);
    issue(n_cur, sub_cur, mk_cur, sK0, sV0, sDoc0);
  }
  for (int st = 0; st < nstages; st += 2) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this lane's DMA landed
    __syncthreads();                     // every lane's DMA landed; buffer 1 free
    if (st + 1 < nstages) {
      next_stage(n_nxt, sub_nxt, mk_nxt);
      issue(n_nxt, sub_nxt, mk_nxt, sK1, sV1, sDoc1);
    }
    compute(n_cur, sub_cur, mk_cur, sK0, sV0, sDoc0);
    if (st + 1 >= nstages) break;
    n_cur = n_nxt;
    sub_cur = sub_nxt;
    mk_cur = mk_nxt;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (st + 2 < nstages) {
      next_stage(n_nxt, sub_nxt, mk_nxt);
      issue(n_nxt, sub_nxt, mk_nxt, sK0, sV0, sDoc0);
    }
    compute(n_cur, sub_cur, mk_cur, sK1, sV1, sDoc1);
    n_cur = n_nxt;
    sub_cur = sub_nxt;
    mk_cur = mk_nxt;
  }

  constexpr float gs = SCORE == FA_SCORE_SOFTCAP ? kSoftcapGrad : 1.0f;
  if (i_ok && p.nsplit > 1) {
    // this part's sum without the scale; the parts are added in order
    // afterwards
    float* po = bp.part_dq + (static_cast<int64_t>(w.c) * p.B * p.H * p.q_len + orow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(po + dt * 32 + 8 * q4 + 4 * g) =
            f32x4{dq[dt][4 * q4 + 0] * gs, dq[dt][4 * q4 + 1] * gs, dq[dt][4 * q4 + 2] * gs,
                  dq[dt][4 * q4 + 3] * gs};
  } else if (i_ok) {
    __bf16* out = static_cast<__bf16*>(bp.dq) + orow * D;
    const float sq = p.scale * gs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = {dq[dt][4 * q4 + 0] * sq, dq[dt][4 * q4 + 1] * sq,
                          dq[dt][4 * q4 + 2] * sq, dq[dt][4 * q4 + 3] * sq};
        *reinterpret_cast<bf16x4*>(out + dt * 32 + 8 * q4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
      }
  }
}

// ------------------------------------------------------------- dK, dV
// The kernel's BwdLaunch argument read from the kernel argument segment
// through a pointer the compiler cannot see through: fields used once per
// stage are fresh scalar loads (scalar cache hits) instead of values held in
// scalar registers across the stage loop, which at one wave per SIMD with
// the accumulators resident would otherwise spill.
typedef const __attribute__((address_space(4))) BwdLaunch KBArgs;
__device__ __forceinline__ KBArgs& kbargs() {
  KBArgs* q = (KBArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(q));
  return *q;
}

template <int D, int BQ, int BK, int SCORE>
__global__ __launch_bounds__(BK * 2, 1) void bwd_dkdv_kernel(const BwdLaunch bp) {
  constexpr int NW = BK / 32;
  constexpr int NT = NW * 64;
  // query rows per stage: the whole 128-row query block for 128-key
  // workgroups (one per CU, so LDS holds two 64 KB stage buffers, and the
  // per-stage fixed cost of DMA issue, list walk and barrier is paid once per
  // 128 rows), else 64 (smaller workgroups keep two per CU)
  constexpr int SR = BQ >= 128 && BK >= 128 ? 128 : kStageKeys;
  constexpr int SPB = BQ / SR;  // stages per query block
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPK = 1024 / RB;
  constexpr int STAGE_BYTES = SR * RB;
  constexpr int ROUNDS = STAGE_BYTES / (NT * 16);
  constexpr int DK = D / 16;
  constexpr int DT = D / 32;
  // one LDS array: per buffer, per query row of the stage its exponent
  // offset, delta and document id, then the Q and dO tiles (1 KB aligned).
  // Every read of the first buffer is a lane offset plus an immediate below
  // 64 KB (the ds_read offset field); with 128-row stages the second buffer
  // lies beyond that and its lane offsets are formed once per stage.
  constexpr int OFF_L = 0, OFF_E = SR * 4, OFF_D = 2 * SR * 4;
  constexpr int OFF_Q = (3 * SR * 4 + 1023) / 1024 * 1024, OFF_O = OFF_Q + STAGE_BYTES;
  constexpr int BUF = OFF_O + STAGE_BYTES;
  constexpr int BUF1 = (BUF + 1023) / 1024 * 1024;  // second buffer, 1 KB aligned
  constexpr int MAX_IMM = OFF_O + (SR - 16) * RB;  // largest immediate of a tile read
  static_assert(MAX_IMM < 65536, "first buffer's reads within the ds_read offset range");
  __shared__ __attribute__((aligned(1024))) char smem[BUF1 + BUF];

  int b, hk, n, c;
  if (!xcd_kv_item(kbargs().f, kbargs().kv_splits, b, hk, n, c)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  int j, dj;  // this lane's key and its document id
  bool j_ok;
  unsigned ispan;
  int ilo;
  bf16x8 kf[DK], vf[DK];  // K^T and V^T as MFMA B operands
  int64_t qstride;
  {
    KBArgs& P = kbargs();
    const int kv_len = P.f.kv_len, q_len = P.f.q_len;
    j = n * BK + wave * 32 + lq;
    j_ok = j < kv_len;
    const int mkind = P.f.mask.kind;
    const int window = P.f.mask.window;
    dj = mkind == FA_MASK_DOCUMENT
             ? P.f.mask.doc_id[static_cast<int64_t>(b) * P.f.mask.doc_stride + (j_ok ? j : 0)]
             : 0;
    // column = key lq, k slots d in [16dk + 8g, +8)
    const __bf16* kr = static_cast<const __bf16*>(P.f.k) + b * P.f.ks[0] + hk * P.f.ks[1] +
                       static_cast<int64_t>(j_ok ? j : 0) * P.f.ks[2];
    const __bf16* vr = static_cast<const __bf16*>(P.f.v) + b * P.f.vs[0] + hk * P.f.vs[1] +
                       static_cast<int64_t>(j_ok ? j : 0) * P.f.vs[2];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      kf[dk] = __builtin_bit_cast(bf16x8, j_ok ? *reinterpret_cast<const u32x4*>(kr + dk * 16 + g * 8) : z);
      vf[dk] = __builtin_bit_cast(bf16x8, j_ok ? *reinterpret_cast<const u32x4*>(vr + dk * 16 + g * 8) : z);
    }
    // mask_mod as an interval of query rows per key: i in [ilo, ilo + ispan)
    // (the end of the sequence is part of the interval)
    const int ihi =
        !j_ok ? 0
        : mkind == FA_MASK_SLIDING_WINDOW || mkind == FA_MASK_LOCAL_WINDOW
            ? static_cast<int>(min(static_cast<int64_t>(j) + window, static_cast<int64_t>(q_len)))
            : q_len;
    ilo = mkind == FA_MASK_LOCAL_WINDOW
              ? static_cast<int>(max(static_cast<int64_t>(j) - window + 1, static_cast<int64_t>(0)))
          : mkind == FA_MASK_NONE ? 0
                                  : j;
    ispan = static_cast<unsigned>(max(ihi - ilo, 0));
    qstride = P.f.qs[2] * 2;  // bytes
  }

  int k_rd[DK];  // row lq (+32 it) of a Q / dO tile as the A operand
  {
    const int sw = kv_swizzle<D>(lq);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) k_rd[dk] = lq * RB + (((2 * dk + g) ^ sw) << 4);
  }
  int v_rd[2][DT];  // transposed reads of a Q / dO tile
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int r = 8 * t2 + 4 * g + ((lane & 15) >> 2);
    const int sw = kv_swizzle<D>(r);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      v_rd[t2][dt] = r * RB + (((d >> 3) ^ sw) << 4) + ((d & 7) << 1);
    }
  }
  uint32_t dma_q[ROUNDS], dma_o[ROUNDS];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int r = (rd * NW + wave) * RPK + lane / CPR;
    const uint32_t col = static_cast<uint32_t>(((lane % CPR) ^ kv_swizzle<D>(r)) * 16);
    dma_q[rd] = static_cast<uint32_t>(r * qstride) + col;
    dma_o[rd] = static_cast<uint32_t>(r * (D * 2)) + col;
  }

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): setup loads landed

  // The block visits of every query head of the group form one flat
  // sequence (head by head; per head its partial list, then its full list),
  // walked by one loop so that the dK / dV accumulators stay in place across
  // heads; a visit is SPB stages of SR rows. Cursor: head cg of the group, its
  // list counts, the next visit of that head.
  int cg = -1, c_np = 0, c_nf = 0, c_it = 0;
  auto head_counts = [&](int gi, int& np, int& nf) {
    KBArgs& P = kbargs();
    const int group = P.f.H / P.f.H_kv;
    const int hh = P.f.Hm == 1 ? 0 : hk * group + gi;
    const int64_t col = (static_cast<int64_t>(P.f.Bm == 1 ? 0 : b) * P.f.Hm + hh) * P.f.nkvb + n;
    np = min(max(((const const_i32*)P.qnum)[col], 0), P.f.nqb);
    nf = P.fqnum ? min(max(((const const_i32*)P.fqnum)[col], 0), P.f.nqb) : 0;
  };
  int total;  // stages of this part
  {
    KBArgs& P = kbargs();
    const int group = P.f.H / P.f.H_kv;
    const int nsplit = P.kv_splits;
    int all_blocks = 0;
    for (int gi = 0; gi < group; ++gi) {
      int np, nf;
      head_counts(gi, np, nf);
      all_blocks += np + nf;
    }
    // part c of nsplit: block visits [v0, v0 + nvis) of the sequence
    const int per_part = (all_blocks + nsplit - 1) / nsplit;
    const int v0 = min(c * per_part, all_blocks);
    total = min(per_part, all_blocks - v0) * SPB;
    // skip the visits of the earlier parts
    int skip = v0;
    while (skip > 0) {
      if (c_it == c_np + c_nf) {
        ++cg;
        head_counts(cg, c_np, c_nf);
        c_it = 0;
        continue;
      }
      const int t = min(skip, c_np + c_nf - c_it);
      skip -= t;
      c_it += t;
    }
  }
  // the next visit: query block m (-1: an index outside [0, NQB), skipped),
  // head h, and whether mask_mod applies. Called once per visit, so a head
  // with visits left always exists.
  auto next_visit = [&](int& m, int& h, bool& masked) {
    while (c_it == c_np + c_nf) {
      ++cg;
      head_counts(cg, c_np, c_nf);
      c_it = 0;
    }
    KBArgs& P = kbargs();
    const int group = P.f.H / P.f.H_kv;
    const int nqb = P.f.nqb;
    const int hh = P.f.Hm == 1 ? 0 : hk * group + cg;
    const int64_t col = (static_cast<int64_t>(P.f.Bm == 1 ? 0 : b) * P.f.Hm + hh) * P.f.nkvb + n;
    const bool part = c_it < c_np;
    const int mm = part ? ((const const_i32*)P.qidx)[col * nqb + c_it]
                        : ((const const_i32*)P.fqidx)[col * nqb + c_it - c_np];
    m = static_cast<unsigned>(mm) < static_cast<unsigned>(nqb) ? mm : -1;
    h = hk * group + cg;
    masked = part || (m + 1) * BQ > P.f.q_len || (n + 1) * BK > P.f.kv_len;
    ++c_it;
  };

  // DMA of stage (m, h, sub) into the buffer at LDS byte offset `buf`
  auto issue = [&](int m, int h, int sub, int buf, bool masked) {
    if (m < 0) return;
    KBArgs& P = kbargs();
    const int q_len = P.f.q_len;
    const char* qbase = reinterpret_cast<const char*>(
        static_cast<const __bf16*>(P.f.q) + b * P.f.qs[0] + h * P.f.qs[1]);
    const int64_t rowbase = (static_cast<int64_t>(b) * P.f.H + h) * q_len;  // dO, LSE, delta
    const char* obase =
        reinterpret_cast<const char*>(static_cast<const __bf16*>(P.dout) + rowbase * D);
    const int i0 = m * BQ + sub * SR;
    const int rows_left = q_len - i0;
    const int qrec = rows_left >= SR ? 0x7fffffff
                     : rows_left <= 0       ? 0
                                            : (rows_left - 1) * static_cast<int>(qstride) + RB;
    const int orec = rows_left >= SR ? 0x7fffffff
                     : rows_left <= 0       ? 0
                                            : (rows_left - 1) * (D * 2) + RB;
    const hw::i32x4 qr = hw::make_rsrc(qbase + (rows_left > 0 ? i0 * qstride : 0), qrec);
    const hw::i32x4 orr = hw::make_rsrc(obase + (rows_left > 0 ? static_cast<int64_t>(i0) * (D * 2) : 0), orec);
    const uint32_t lb = hw::opaque_u32(hw::lds_addr(smem) + buf) + wave * 1024;
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      hw::dma_tile16(qr, lb + OFF_Q + rd * NW * 1024, dma_q[rd], 0);
      hw::dma_tile16(orr, lb + OFF_O + rd * NW * 1024, dma_o[rd], 0);
    }
    if (wave < SR / 64) {  // one wave per 64 rows of the stage
      const uint32_t lr = hw::opaque_u32(hw::lds_addr(smem) + buf) + wave * 256;
      const uint32_t r4 = static_cast<uint32_t>(min(i0 + wave * 64 + lane, q_len - 1)) * 4;
      hw::dma_dword(reinterpret_cast<const int*>(P.rowterm + rowbase), lr + OFF_L, r4);
      hw::dma_dword(reinterpret_cast<const int*>(P.delta + rowbase), lr + OFF_E, r4);
      if (masked && P.f.mask.kind == FA_MASK_DOCUMENT)
        hw::dma_dword(P.f.mask.doc_id + static_cast<int64_t>(b) * P.f.mask.doc_stride,
                      lr + OFF_D, r4);
    }
  };

  // score constants: those that do not depend on the head once; ALiBi's key
  // term slope_h log2e j formed again only when the head changes (the
  // stages of one head follow each other)
  const ScoreConsts sc = make_score_consts(kbargs().f, 0);
  float tj = 0.0f;
  int tj_h = -1;
  auto compute = [&](auto second, int m, int h, int sub, bool masked) {
    if (m < 0) return;
    // lane offsets into this stage's buffer (see the LDS layout above)
    constexpr int BO = decltype(second)::value ? BUF1 : 0;
    constexpr bool far = BO + MAX_IMM >= 65536;
    constexpr int BI = far ? 0 : BO;  // buffer offset left in the immediates
    int kq[DK], vq[2][DT];
#pragma unroll
    for (int dd = 0; dd < DK; ++dd) kq[dd] = far ? opaque_v(k_rd[dd] + BO) : k_rd[dd];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vq[t2][dt] = far ? opaque_v(v_rd[t2][dt] + BO) : v_rd[t2][dt];
    const int rq = far ? opaque_v(BO + 16 * g) : 16 * g;  // row terms of rows 4g..
    const char* sQ = smem + BI + OFF_Q;
    const char* sO = smem + BI + OFF_O;
    const float* sL = reinterpret_cast<const float*>(smem + BI + OFF_L + rq);
    const float* sE = reinterpret_cast<const float*>(smem + BI + OFF_E + rq);
    const int* sD = reinterpret_cast<const int*>(smem + BI + OFF_D + rq);
    if constexpr (SCORE == FA_SCORE_ALIBI) {
      if (h != tj_h) {
        tj = make_score_consts(kbargs().f, h).slope2 * static_cast<float>(j);
        tj_h = h;
      }
    }
    const int i0 = m * BQ + sub * SR;

    // Parts of 32 query rows each (it), one after the other: the live fp32
    // tiles per part are one S and one dP tile, which leaves the compiler
    // registers to keep several LDS reads in flight.
#pragma unroll
    for (int it = 0; it < SR / 32; ++it) {
      // S = Q K^T and dP = dO V^T for rows [32 it, 32 it + 32) of the stage
      f32x16 s = f32x16{}, dpm = f32x16{};
      u32x4 qa[DK], oa[DK];
#pragma unroll
      for (int dd = 0; dd < DK; ++dd) {
        qa[dd] = *reinterpret_cast<const u32x4*>(sQ + kq[dd] + it * 32 * RB);
        oa[dd] = *reinterpret_cast<const u32x4*>(sO + kq[dd] + it * 32 * RB);
      }
#pragma unroll
      for (int dd = 0; dd < DK; ++dd) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[dd]), kf[dd],
                                                    s, 0, 0, 0);
        dpm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, oa[dd]), vf[dd],
                                                      dpm, 0, 0, 0);
      }

      // element r: query row i0 + 32 it + 8 (r / 4) + 4 g + r % 4. The
      // row's exponent offset (rowterm, from the dQ kernel) folds in -LSE
      // and ALiBi's row part; the key part of ALiBi is tj.
      float fp[16];  // score_mod' (soft-cap), else 1
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int il = 32 * it + 8 * r4;  // + 4g: first of 4 consecutive rows
        const f32x4 rt4 = *reinterpret_cast<const f32x4*>(sL + il);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int r = 4 * r4 + cc;
          float arg;
          fp[r] = 1.0f;
          if constexpr (SCORE == FA_SCORE_ALIBI) {
            arg = __builtin_fmaf(s[r], sc.c, rt4[cc] + tj);
          } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
            const float e = exp2_hw(s[r] * (2.0f * sc.cap_in * kLog2e));
            const float tt = __builtin_amdgcn_rcpf(e + 1.0f);
            arg = __builtin_fmaf(-2.0f * sc.cap_out, tt, sc.cap_out + rt4[cc]);
            fp[r] = __builtin_fmaf(-tt, tt, tt);  // (1 - tanh^2) / 4
          } else {
            arg = __builtin_fmaf(s[r], sc.c, rt4[cc]);
          }
          s[r] = exp2_hw(arg);  // P
        }
      }
      // mask_mod on partial and tail stages only (a uniform branch)
      if (masked) {
        const int q_len = kbargs().f.q_len;
        const bool doc_mask = kbargs().f.mask.kind == FA_MASK_DOCUMENT;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int il = 32 * it + 8 * r4;  // + 4g
          int4 d4 = {dj, dj, dj, dj};
          if (doc_mask) d4 = *reinterpret_cast<const int4*>(sD + il);
          const int dqs[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const int irow = i0 + il + 4 * g + cc;
            const bool ok =
                (static_cast<unsigned>(irow - ilo) < ispan) & (dqs[cc] == dj) & (irow < q_len);
            s[4 * r4 + cc] = ok ? s[4 * r4 + cc] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 del4 = *reinterpret_cast<const f32x4*>(sE + 32 * it + 8 * r4);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int r = 4 * r4 + cc;
          dpm[r] = s[r] * (dpm[r] - del4[cc]) * fp[r];  // dT
        }
      }
      bf16x8 pb[2], tb[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x8 pf, tf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[e] = s[h2 * 8 + e];
          tf[e] = dpm[h2 * 8 + e];
        }
        pb[h2] = __builtin_convertvector(pf, bf16x8);
        tb[h2] = __builtin_convertvector(tf, bf16x8);
      }

      // dV^T += dO^T P and dK^T += Q^T dT over these 32 rows (2 k-steps
      // of 16)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int kk = 2 * it + h2;
        i16x8 o8[DT], q8[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const i16x4 olo = lds_read_tr(sO + vq[0][dt] + kk * 16 * RB);
          const i16x4 ohi = lds_read_tr(sO + vq[1][dt] + kk * 16 * RB);
          o8[dt] = i16x8{olo[0], olo[1], olo[2], olo[3], ohi[0], ohi[1], ohi[2], ohi[3]};
          const i16x4 qlo = lds_read_tr(sQ + vq[0][dt] + kk * 16 * RB);
          const i16x4 qhi = lds_read_tr(sQ + vq[1][dt] + kk * 16 * RB);
          q8[dt] = i16x8{qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o8[dt]),
                                                           pb[h2], dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q8[dt]),
                                                           tb[h2], dk[dt], 0, 0, 0);
        }
      }
    }
  };

  // Stage loop, unrolled by two so that each LDS buffer is addressed with
  // constant offsets; the DMA of stage st + 1 overlaps the compute of stage
  // st. (m, h, masked): the visit of the stage; sub: its 64-row part.
  int c_m = -1, c_h = 0, c_sub = 0;
  bool c_mk = false;
  auto next_stage = [&](int& m, int& h, int& sub, bool& masked) {
    if (c_sub == 0) next_visit(c_m, c_h, c_mk);
    m = c_m;
    h = c_h;
    sub = c_sub;
    masked = c_mk;
    if (++c_sub == SPB) c_sub = 0;
  };
  int m_cur = -1, h_cur = 0, sub_cur = 0, m_nxt = -1, h_nxt = 0, sub_nxt = 0;
  bool mk_cur = false, mk_nxt = false;
  if (total > 0) {
    next_stage(m_cur, h_cur, sub_cur, mk_cur);
    issue(m_cur, h_cur, sub_cur, 0, mk_cur);
  }
  for (int st = 0; st < total; st += 2) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this lane's DMA landed
    __syncthreads();                     // every lane's DMA landed; buffer 1 free
    if (st + 1 < total) {
      next_stage(m_nxt, h_nxt, sub_nxt, mk_nxt);
      issue(m_nxt, h_nxt, sub_nxt, BUF1, mk_nxt);
    }
    compute(std::false_type{}, m_cur, h_cur, sub_cur, mk_cur);
    if (st + 1 >= total) break;
    m_cur = m_nxt;
    h_cur = h_nxt;
    sub_cur = sub_nxt;
    mk_cur = mk_nxt;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (st + 2 < total) {
      next_stage(m_nxt, h_nxt, sub_nxt, mk_nxt);
      issue(m_nxt, h_nxt, sub_nxt, 0, mk_nxt);
    }
    compute(std::true_type{}, m_cur, h_cur, sub_cur, mk_cur);
    m_cur = m_nxt;
    h_cur = h_nxt;
    sub_cur = sub_nxt;
    mk_cur = mk_nxt;
  }

  KBArgs& P = kbargs();
  const int kv_len = P.f.kv_len;
  constexpr float gs = SCORE == FA_SCORE_SOFTCAP ? kSoftcapGrad : 1.0f;
  if (j_ok && P.kv_splits > 1) {
    // this part's sums without the scale; the parts are added in order
    // afterwards
    const int64_t krow = (static_cast<int64_t>(b) * P.f.H_kv + hk) * kv_len + j;
    const int64_t prow = static_cast<int64_t>(c) * P.f.B * P.f.H_kv * kv_len + krow;
    float* pk = P.part_dk + prow * D;
    float* pv = P.part_dv + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        *reinterpret_cast<f32x4*>(pk + dt * 32 + 8 * q4 + 4 * g) =
            f32x4{dk[dt][4 * q4 + 0] * gs, dk[dt][4 * q4 + 1] * gs, dk[dt][4 * q4 + 2] * gs,
                  dk[dt][4 * q4 + 3] * gs};
        *reinterpret_cast<f32x4*>(pv + dt * 32 + 8 * q4 + 4 * g) =
            f32x4{dv[dt][4 * q4 + 0], dv[dt][4 * q4 + 1], dv[dt][4 * q4 + 2], dv[dt][4 * q4 + 3]};
      }
  } else if (j_ok) {
    const int64_t krow = (static_cast<int64_t>(b) * P.f.H_kv + hk) * kv_len + j;
    __bf16* outk = static_cast<__bf16*>(P.dk) + krow * D;
    __bf16* outv = static_cast<__bf16*>(P.dv) + krow * D;
    const float scale = P.f.scale * gs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 k4 = {dk[dt][4 * q4 + 0] * scale, dk[dt][4 * q4 + 1] * scale,
                          dk[dt][4 * q4 + 2] * scale, dk[dt][4 * q4 + 3] * scale};
        const f32x4 v4 = {dv[dt][4 * q4 + 0], dv[dt][4 * q4 + 1], dv[dt][4 * q4 + 2],
                          dv[dt][4 * q4 + 3]};
        *reinterpret_cast<bf16x4*>(outk + dt * 32 + 8 * q4 + 4 * g) = __builtin_convertvector(k4, bf16x4);
        *reinterpret_cast<bf16x4*>(outv + dt * 32 + 8 * q4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
      }
  }
}

}  // namespace fa
