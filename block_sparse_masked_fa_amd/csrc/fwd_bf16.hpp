// Fused block-sparse attention forward, bf16 inputs, fp32 accumulation, on
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes one query block (BLK rows) of one head; BLK / 32
// wavefronts each own 32 query rows. For every live key block of the row's
// lists (full blocks first, then partial ones) the workgroup:
//   1. stages the K tile [BLK keys][D] and the V tile, transposed to
//      [D][BLK keys], in LDS from 16-byte coalesced global loads;
//   2. computes S^T = K Q^T on MFMA. With keys on the MFMA row axis and
//      queries on the column axis, each lane's 16 accumulator values belong
//      to ONE query (column lane % 32), so a query row is spread over only
//      two lanes (l and l + 32): row statistics are in-lane reductions plus
//      one cross-half exchange;
//   3. applies score_mod to every position and, on partial blocks only, the
//      mask_mod (full blocks skip it: tensorplay create_block_mask page,
//      separate_full_blocks);
//   4. updates the online softmax (running max m, running sum l, rescale of
//      the output accumulator by exp2(m_old - m_new)), so no score matrix is
//      ever stored;
//   5. rounds P to bf16 and accumulates O^T += V^T P^T on MFMA. The P values
//      of step 2's accumulator are already laid out as the MFMA B operand;
//      the MFMA contracts over its k slots in any consistent order, so the V^T
//      tile is stored with keys permuted inside each group of 16 so that a
//      lane's 8 slots are one 16-byte LDS read.
// The epilogue writes O = acc / l (bf16) and LSE = m + ln l (fp32).
#pragma once

#include "fwd_common.hpp"

namespace fa {

template <int D, int BLK, int SCORE>
__global__ __launch_bounds__(BLK * 2, 2) void fwd_bf16_kernel(const FwdLaunch p) {
  constexpr int NT = BLK * 2;     // threads: BLK / 32 waves of 64
  constexpr int JT = BLK / 32;    // 32-key MFMA tiles per key block
  constexpr int DK = D / 16;      // k-steps of QK^T
  constexpr int DT = D / 32;      // 32-wide d tiles of the output
  constexpr int KS = BLK / 16;    // k-steps of PV
  constexpr int KST = D + 8;      // LDS row stride of K (elements)
  constexpr int VST = BLK + 8;    // LDS row stride of V^T (elements)

  __shared__ __attribute__((aligned(16))) __bf16 sK[BLK * KST];
  __shared__ __attribute__((aligned(16))) __bf16 sV[D * VST];
  __shared__ int sDoc[BLK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  const WorkItem w = work_item(p);
  const int hk = w.h / (p.H / p.H_kv);
  const int i = w.m * BLK + wave * 32 + lq;  // this lane's query row
  const bool i_ok = i < p.q_len;
  const int kv_len = p.kv_len;
  const int mkind = p.mask.kind;
  const int window = p.mask.window;
  const int* doc = p.mask.doc_id;

  const __bf16* qp = static_cast<const __bf16*>(p.q) + w.b * p.qs[0] + w.h * p.qs[1];
  const __bf16* kp = static_cast<const __bf16*>(p.k) + w.b * p.ks[0] + hk * p.ks[1];
  const __bf16* vp = static_cast<const __bf16*>(p.v) + w.b * p.vs[0] + hk * p.vs[1];
  const int64_t ks2 = p.ks[2];
  const int64_t vs2 = p.vs[2];

  // Q^T as the MFMA B operand: column = query lq, k slots = d in
  // [dk*16 + g*8, +8).
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
  const int di = (mkind == FA_MASK_DOCUMENT) ? doc[i_ok ? i : 0] : 0;

  // The row's block lists (broadcast over batch / head when Bm / Hm is 1).
  const int bb = p.Bm == 1 ? 0 : w.b;
  const int hh = p.Hm == 1 ? 0 : w.h;
  const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + w.m;
  const int nkvb = p.nkvb;
  const int nf = p.fnum ? min(max(p.fnum[lrow], 0), nkvb) : 0;
  const int np = min(max(p.num[lrow], 0), nkvb);
  const int32_t* fl = p.fidx ? p.fidx + lrow * nkvb : nullptr;
  const int32_t* pl = p.idx + lrow * nkvb;

  const ScoreConsts sc = make_score_consts(p, w.h);

  float m_run = FA_NEG_INF;  // running max, log2 domain
  float l_run = 0.0f;        // this lane's share of the running sum
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  for (int it = 0; it < nf + np; ++it) {
    const bool from_full = it < nf;
    const int n = from_full ? fl[it] : pl[it - nf];
    if (static_cast<unsigned>(n) >= static_cast<unsigned>(nkvb)) continue;
    const int j0 = n * BLK;
    const bool masked = !from_full || (j0 + BLK > kv_len);

    __syncthreads();  // previous tile fully consumed
    // ---- stage K [BLK][D]
#pragma unroll
    for (int c = tid; c < BLK * (D / 8); c += NT) {
      const int r = c / (D / 8);
      const int cc = c % (D / 8);
      const int j = j0 + r;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (j < kv_len) x = *reinterpret_cast<const u32x4*>(kp + j * ks2 + cc * 8);
      *reinterpret_cast<u32x4*>(&sK[r * KST + cc * 8]) = x;
    }
    // ---- stage V^T [D][BLK] with the in-group key permutation: key
    // 16G + 8a + 4s + c sits at column 16G + 8s + 4a + c.
#pragma unroll
    for (int t = tid; t < (BLK / 8) * (D / 8); t += NT) {
      const int dc = t % (D / 8);
      const int js = t / (D / 8);
      const int G = js >> 1;
      const int sg = js & 1;
      u32x4 rv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = j0 + 16 * G + 4 * sg + (r & 3) + 8 * (r >> 2);
        rv[r] = u32x4{0u, 0u, 0u, 0u};
        if (j < kv_len) rv[r] = *reinterpret_cast<const u32x4*>(vp + j * vs2 + dc * 8);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        u32x4 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t x = rv[2 * u][tt >> 1];
          const uint32_t y = rv[2 * u + 1][tt >> 1];
          o[u] = (tt & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
        *reinterpret_cast<u32x4*>(&sV[(dc * 8 + tt) * VST + 16 * G + 8 * sg]) = o;
      }
    }
    if (masked && mkind == FA_MASK_DOCUMENT) {
      for (int t = tid; t < BLK; t += NT) sDoc[t] = (j0 + t < kv_len) ? doc[j0 + t] : -1;
    }
    __syncthreads();

    // ---- S^T = K Q^T
    f32x16 s[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) s[jt] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sK[(jt * 32 + lq) * KST + dk * 16 + g * 8]);
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[dk],
                                                        s[jt], 0, 0, 0);
      }
    }

    // ---- score_mod on every position; key of (jt, r) is
    // j0 + 4g + jt*32 + 8*(r/4) + r%4
    const float ibase = static_cast<float>(i - j0 - 4 * g);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[jt][r] = score2<SCORE>(s[jt][r], sc,
                                 ibase - static_cast<float>(jt * 32 + 8 * (r >> 2) + (r & 3)));

    // ---- mask_mod on partial (and sequence-tail) blocks only
    if (masked) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 4 * g + jt * 32 + 8 * (r >> 2) + (r & 3);
          const int j = j0 + jl;
          bool ok = j < kv_len;
          switch (mkind) {
            case FA_MASK_CAUSAL: ok &= mask_ok<FA_MASK_CAUSAL>(i, j, window, di, 0); break;
            case FA_MASK_SLIDING_WINDOW: ok &= mask_ok<FA_MASK_SLIDING_WINDOW>(i, j, window, di, 0); break;
            case FA_MASK_DOCUMENT: ok &= mask_ok<FA_MASK_DOCUMENT>(i, j, window, di, sDoc[jl]); break;
            default: break;
          }
          s[jt][r] = ok ? s[jt][r] : FA_NEG_INF;
        }
    }

    // ---- online softmax
    float mx = FA_NEG_INF;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[jt][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m_run, mx);
    const float m_use = (m_new == FA_NEG_INF) ? 0.0f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    m_run = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_hw(s[jt][r] - m_use);
        s[jt][r] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const f32x16& src = s[kk >> 1];
      const int h8 = (kk & 1) * 8;
      const f32x8 pf = {src[h8 + 0], src[h8 + 1], src[h8 + 2], src[h8 + 3],
                        src[h8 + 4], src[h8 + 5], src[h8 + 6], src[h8 + 7]};
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&sV[(dt * 32 + lq) * VST + kk * 16 + g * 8]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb,
                                                           oacc[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (i_ok) {
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
