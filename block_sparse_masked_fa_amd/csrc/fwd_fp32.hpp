// Fused block-sparse attention forward in fp32 on gfx950 MFMA
// (v_mfma_f32_32x32x2_f32). Same structure as the bf16 kernel (one workgroup
// per query block, one wavefront per 32 queries, S^T = K Q^T so each lane
// owns one query, online softmax, O^T += V^T P^T), with everything in fp32:
// P is never rounded. A 32x32x2 MFMA takes a single k value per lane, so
// V's B-operand reads are one float per lane from the row-major V tile and
// no transpose is needed.
#pragma once

#include "fwd_common.hpp"

namespace fa {

template <int D, int BLK, int SCORE>
__global__ __launch_bounds__(BLK * 2) void fwd_fp32_kernel(const FwdLaunch p) {
  constexpr int NT = BLK * 2;
  constexpr int JT = BLK / 32;
  constexpr int DT = D / 32;
  constexpr int ST = D + 4;  // LDS row stride (floats)

  __shared__ __attribute__((aligned(16))) float sK[BLK * ST];
  __shared__ __attribute__((aligned(16))) float sV[BLK * ST];
  __shared__ int sDoc[BLK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  const WorkItem w = work_item(p);
  const int hk = w.h / (p.H / p.H_kv);
  const int i = w.m * BLK + wave * 32 + lq;
  const bool i_ok = i < p.q_len;
  const int kv_len = p.kv_len;
  const int mkind = p.mask.kind;
  const int window = p.mask.window;
  const int* doc = p.mask.doc_id + static_cast<int64_t>(w.b) * p.mask.doc_stride;

  const float* qp = static_cast<const float*>(p.q) + w.b * p.qs[0] + w.h * p.qs[1];
  const float* kp = static_cast<const float*>(p.k) + w.b * p.ks[0] + hk * p.ks[1];
  const float* vp = static_cast<const float*>(p.v) + w.b * p.vs[0] + hk * p.vs[1];

  // Q^T B operand: column = query lq, k slot g of step t is d = 2t + g.
  float qf[D / 2];
  {
    const float* row = qp + static_cast<int64_t>(i_ok ? i : 0) * p.qs[2];
#pragma unroll
    for (int t = 0; t < D / 2; ++t) qf[t] = i_ok ? row[2 * t + g] : 0.0f;
  }
  const int di = (mkind == FA_MASK_DOCUMENT) ? doc[i_ok ? i : 0] : 0;

  const int bb = p.Bm == 1 ? 0 : w.b;
  const int hh = p.Hm == 1 ? 0 : w.h;
  const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + w.m;
  const int nkvb = p.nkvb;
  const int nf = p.fnum ? min(max(p.fnum[lrow], 0), nkvb) : 0;
  const int np = min(max(p.num[lrow], 0), nkvb);
  const int32_t* fl = p.fidx ? p.fidx + lrow * nkvb : nullptr;
  const int32_t* pl = p.idx + lrow * nkvb;

  const ScoreConsts sc = make_score_consts(p, w.h);

  float m_run = FA_NEG_INF;
  float l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  for (int it = 0; it < nf + np; ++it) {
    const bool from_full = it < nf;
    const int n = from_full ? fl[it] : pl[it - nf];
    if (static_cast<unsigned>(n) >= static_cast<unsigned>(nkvb)) continue;
    const int j0 = n * BLK;
    const bool masked = !from_full || (j0 + BLK > kv_len);

    __syncthreads();
    for (int c = tid; c < BLK * (D / 4); c += NT) {
      const int r = c / (D / 4);
      const int cc = c % (D / 4);
      const int j = j0 + r;
      f32x4 xk = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 xv = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < kv_len) {
        xk = *reinterpret_cast<const f32x4*>(kp + j * p.ks[2] + cc * 4);
        xv = *reinterpret_cast<const f32x4*>(vp + j * p.vs[2] + cc * 4);
      }
      *reinterpret_cast<f32x4*>(&sK[r * ST + cc * 4]) = xk;
      *reinterpret_cast<f32x4*>(&sV[r * ST + cc * 4]) = xv;
    }
    if (masked && mkind == FA_MASK_DOCUMENT) {
      for (int t = tid; t < BLK; t += NT) sDoc[t] = (j0 + t < kv_len) ? doc[j0 + t] : -1;
    }
    __syncthreads();

    f32x16 s[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) s[jt] = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 2; ++t)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[(jt * 32 + lq) * ST + 2 * t + g], qf[t],
                                                     s[jt], 0, 0, 0);

    const float ibase = static_cast<float>(i - j0 - 4 * g);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[jt][r] = score2<SCORE>(s[jt][r], sc,
                                 ibase - static_cast<float>(jt * 32 + 8 * (r >> 2) + (r & 3)));

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
            case FA_MASK_LOCAL_WINDOW: ok &= mask_ok<FA_MASK_LOCAL_WINDOW>(i, j, window, di, 0); break;
            case FA_MASK_DOCUMENT: ok &= mask_ok<FA_MASK_DOCUMENT>(i, j, window, di, sDoc[jl]); break;
            default: break;
          }
          s[jt][r] = ok ? s[jt][r] : FA_NEG_INF;
        }
    }

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

    // O^T += V^T P^T: step (jt, r) pairs k slot g with key
    // jt*32 + 8*(r/4) + 4g + r%4, which is exactly the key of this lane's
    // accumulator value s[jt][r].
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = jt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[jl * ST + dt * 32 + lq], s[jt][r],
                                                          oacc[dt], 0, 0, 0);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (i_ok) {
    const int64_t orow = (static_cast<int64_t>(w.b) * p.H + w.h) * p.q_len + i;
    float* op = static_cast<float*>(p.o) + orow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = {oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv,
                          oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * q4 + 4 * g) = v4;
      }
    if (g == 0 && p.lse)
      p.lse[orow] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : FA_NEG_INF;
  }
}

}  // namespace fa
