// Decode step over a paged key/value cache, bf16, for gfx950.
//
// Each sequence b holds L_b cached tokens, the newest one included, in a
// pool of physical pages of page_size token rows; its page table maps
// logical page p (tokens [p * page_size, (p + 1) * page_size)) to a
// physical page (PagedAttention: the key/value cache kept as pages,
// frontiernews "What Attention Patterns Does FlexAttention Support?"). The
// newest token queries at position i = L_b - 1 over keys [0, L_b) under the
// built-in mask_mod and score_mod, as the forward does for one row.
//
// Work split: one single-wavefront workgroup per (sequence, key head, part).
// The wave's 32 MFMA query columns are the query heads of the key head's
// group (grouped heads share the key/value tiles they read; columns past
// the group are zero and never stored). The keys the mask can allow form one
// interval [lo, L_b) (every built-in mask allows only keys at or before the
// query, and the window masks only the last W of them); its 64-key stages
// are cut into `nsplit` consecutive parts, and the parts are merged by the
// split-KV combine kernel. Per stage: the stage's physical address comes
// from the page table (page_size is a multiple of 64, so no stage crosses a
// page); the V tile arrives in LDS by buffer DMA (double-buffered, read
// transposed as in the forward, fwd_bf16.hpp) and K goes straight into
// registers in the MFMA operand layout, which halves the LDS per workgroup
// so that four workgroups (and their loads in flight) fit a compute unit;
// S^T = K Q^T and
// O^T += V^T P^T on MFMA, and an online softmax per query column. mask_mod
// runs on the interval's first and last stage (and on every stage of a
// document mask). A page-table entry outside [0, num_pages) skips its
// stage: those keys are left out.
//
// Roofline: HBM. A sequence's keys and values are read once per step.
#pragma once

#include "fwd_bf16.hpp"

namespace fa {

template <int D, int SCORE>
__global__ __launch_bounds__(64) void decode_paged_kernel(const DecodeLaunch p) {
  constexpr int RB = D * 2;               // bytes per LDS row
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPK = 1024 / RB;          // rows per 1 KB DMA segment
  constexpr int STAGE_BYTES = kStageKeys * RB;
  constexpr int ROUNDS = STAGE_BYTES / (64 * 16);
  constexpr int DK = D / 16;
  constexpr int DT = D / 32;

  __shared__ __attribute__((aligned(1024))) char sV0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int sDoc0[kStageKeys];
  __shared__ __attribute__((aligned(16))) int sDoc1[kStageKeys];

  const int wg = blockIdx.x;
  const int c = wg % p.nsplit;
  const int bh = wg / p.nsplit;
  const int hk = bh % p.H_kv;
  const int b = bh / p.H_kv;
  if (b >= p.B) return;

  const int lane = threadIdx.x;
  const int lq = lane & 31;
  const int g = lane >> 5;
  const int group = p.H / p.H_kv;
  const int h = hk * group + lq;  // this lane's query head (column lq)
  const bool h_ok = lq < group;

  // cached tokens of the sequence (clamped to what its page table can hold)
  const int cap = p.max_pages * p.page_size;
  const int L = min(max(p.seq_lens[b], 0), cap);
  const int i = L - 1;  // the query's position
  const int mkind = p.mask.kind;
  const int window = p.mask.window;
  const int* doc = p.mask.doc_id + static_cast<int64_t>(b) * p.mask.doc_stride;
  const bool doc_mask = mkind == FA_MASK_DOCUMENT;
  // keys the mask can allow: [lo, L)
  const int lo = (mkind == FA_MASK_SLIDING_WINDOW || mkind == FA_MASK_LOCAL_WINDOW)
                     ? static_cast<int>(max(static_cast<int64_t>(i) - window + 1, static_cast<int64_t>(0)))
                     : 0;
  const unsigned span = static_cast<unsigned>(max(L - lo, 0));
  const int st_first = lo / kStageKeys;
  const int st_total = L > 0 ? (L + kStageKeys - 1) / kStageKeys - st_first : 0;
  // this part's stages: [st_first + v0, st_first + v0 + nst)
  const int per_part = (st_total + p.nsplit - 1) / p.nsplit;
  const int v0 = min(c * per_part, st_total);
  const int nst = min(per_part, st_total - v0);

  // Q^T as the MFMA B operand: column lq = head h, k slots d in [16dk + 8g, +8)
  bf16x8 qf[DK];
  {
    const __bf16* row = static_cast<const __bf16*>(p.q) + b * p.qs[0] +
                        static_cast<int64_t>(h_ok ? h : 0) * p.qs[1];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[dk] = __builtin_bit_cast(
          bf16x8, h_ok ? *reinterpret_cast<const u32x4*>(row + dk * 16 + g * 8) : z);
    }
  }
  const int di = doc_mask && L > 0 ? doc[i] : 0;

  // score_mod constants in the log2 domain (per lane: the ALiBi slope
  // belongs to the lane's query head)
  const float sc_c = p.scale * kLog2e;
  const float slope2 =
      SCORE == FA_SCORE_ALIBI
          ? exp2_hw(-8.0f * static_cast<float>(h + 1) / static_cast<float>(p.H)) * kLog2e
          : 0.0f;
  const float cap_in = SCORE == FA_SCORE_SOFTCAP ? p.scale / p.softcap : 0.0f;
  const float cap_out = SCORE == FA_SCORE_SOFTCAP ? p.softcap * kLog2e : 0.0f;

  const char* kpool = reinterpret_cast<const char*>(p.k_pages);
  const char* vpool = reinterpret_cast<const char*>(p.v_pages);
  const int64_t krow = p.ks[1] * 2;  // bytes between token rows of a page
  const int64_t vrow = p.vs[1] * 2;
  const int32_t* table = p.page_table + static_cast<int64_t>(b) * p.max_pages;

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

  // stage k of the part: absolute key offset, physical page (-1: skipped)
  auto stage_j0 = [&](int k) -> int { return (st_first + v0 + k) * kStageKeys; };
  auto stage_page = [&](int k) -> int {
    const int lp = stage_j0(k) / p.page_size;
    const int phys = table[lp];
    return static_cast<unsigned>(phys) < static_cast<unsigned>(p.num_pages) ? phys : -1;
  };
  auto masked_at = [&](int j0) -> bool { return doc_mask || j0 < lo || j0 + kStageKeys > L; };
  auto stage_base = [&](const char* pool, const int64_t* st, int phys, int j0) -> const char* {
    return pool + (static_cast<int64_t>(phys) * st[0] + hk * st[2] +
                   static_cast<int64_t>(j0 % p.page_size) * st[1]) * 2;
  };
  // V tile of stage k into LDS by DMA (rows past the sequence end as zeros)
  auto issue_v = [&](int k, int phys, char* sV, int* sD) {
    if (phys < 0) return;
    const int j0 = stage_j0(k);
    const int rows_left = L - j0;
    const int vrec = rows_left >= kStageKeys ? 0x7fffffff
                     : (rows_left - 1) * static_cast<int>(vrow) + RB;
    const hw::i32x4 vr = hw::make_rsrc(stage_base(vpool, p.vs, phys, j0), vrec);
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int r = rd * RPK + lane / CPR;
      const uint32_t col = static_cast<uint32_t>(((lane % CPR) ^ kv_swizzle<D>(r)) * 16);
      hw::dma_tile16(vr, hw::lds_addr(sV + rd * 1024), static_cast<uint32_t>(r * vrow) + col, 0);
    }
    if (doc_mask) {
      const int j = min(j0 + lane, L - 1);
      hw::dma_dword(doc, hw::lds_addr(sD), static_cast<uint32_t>(j * 4));
    }
  };
  // K of stage k straight into registers, already in the MFMA A-operand
  // layout (row lq + 32 jt, chunk 2 dk + g), by buffer loads whose range
  // ends at the sequence end (rows past it read as zeros)
  u32x4 kreg[DK][2];
  auto load_k = [&](int k, int phys) {
    if (phys < 0) return;
    const int j0 = stage_j0(k);
    const int rows_left = L - j0;
    const int krec = rows_left >= kStageKeys ? 0x7fffffff
                     : (rows_left - 1) * static_cast<int>(krow) + RB;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(stage_base(kpool, p.ks, phys, j0)), 0, krec, hw::kRawBufferFlags);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int vo = (lq + 32 * jt) * static_cast<int>(krow) + g * 16;
#pragma unroll
      for (int dk = 0; dk < DK; ++dk)
        kreg[dk][jt] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, vo + dk * 32, 0, 0));
    }
  };

  float m_run = FA_NEG_INF;  // reference max, log2 domain
  float l_run = 0.0f;
  float l_run2 = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // S^T = K Q^T for the stage's 64 keys (K from registers)
  auto scores = [&](f32x16* s) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kreg[dk][jt]),
                                                        qf[dk], s[jt], 0, 0, 0);
    }
  };
  auto compute = [&](int k, int phys, f32x16* s, const char* sV, const int* sD) {
    if (phys < 0) return;
    const int j0 = stage_j0(k);
    const bool masked = masked_at(j0);

    // score_mod into the log2 domain; key of (jt, r): j0 + 4g + 32jt +
    // 8(r/4) + r%4
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const float bias0 =
          SCORE == FA_SCORE_ALIBI ? slope2 * static_cast<float>(j0 + 4 * g + 32 * jt - i) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (SCORE == FA_SCORE_ALIBI) {
          const float bj = __builtin_fmaf(slope2, static_cast<float>(8 * (r >> 2) + (r & 3)), bias0);
          s[jt][r] = __builtin_fmaf(s[jt][r], sc_c, bj);
        } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
          const float e = exp2_hw(s[jt][r] * (2.0f * cap_in * kLog2e));
          const float t = __builtin_amdgcn_rcpf(e + 1.0f);
          s[jt][r] = __builtin_fmaf(-2.0f * cap_out, t, cap_out);
        } else {
          s[jt][r] *= sc_c;
        }
      }
    }

    // mask_mod on the interval's edge stages (every stage of a document
    // mask): the key interval [lo, L) and the document equality
    if (masked) {
      const int lor = lo - (j0 + 4 * g);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int jl = 32 * jt + 8 * r4;
          int dj[4] = {di, di, di, di};
          if (doc_mask) {
            const int4 t = *reinterpret_cast<const int4*>(sD + 4 * g + jl);
            dj[0] = t.x; dj[1] = t.y; dj[2] = t.z; dj[3] = t.w;
          }
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const bool ok = (static_cast<unsigned>(jl + cc - lor) < span) & (dj[cc] == di);
            s[jt][4 * r4 + cc] = ok ? s[jt][4 * r4 + cc] : FA_NEG_INF;
          }
        }
    }

    // online softmax per query column (lazy rescale, as in the forward)
    float mx4[4] = {FA_NEG_INF, FA_NEG_INF, FA_NEG_INF, FA_NEG_INF};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int r = 0; r < 8; ++r) mx4[q4] = __builtin_fmaxf(mx4[q4], s[q4 >> 1][8 * (q4 & 1) + r]);
    float mx = __builtin_fmaxf(__builtin_fmaxf(mx4[0], mx4[1]), __builtin_fmaxf(mx4[2], mx4[3]));
    mx = row_pair_max(mx);
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
      for (int e = 0; e < 8; ++e) pf[e] = exp2_hw(s[kk >> 1][(kk & 1) * 8 + e] - m_use);
      pb[kk] = __builtin_convertvector(pf, bf16x8);
      const u32x4 pw = __builtin_bit_cast(u32x4, pb[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = pw[e];  // copied out: see fwd_bf16.hpp
        float& acc = (e & 1) ? l_run2 : l_run;
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), ones, acc, false);
      }
    }

    // O^T += V^T P^T (4 k-steps of 16 keys)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 vlo = lds_read_tr(sV + v_rd[0][dt] + kk * 16 * RB);
        const i16x4 vhi = lds_read_tr(sV + v_rd[1][dt] + kk * 16 * RB);
        const i16x8 a8 = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[kk],
                                                           oacc[dt], 0, 0, 0);
      }
    }
  };

  // main loop: stage k + 1's V tile (DMA) and K registers (loaded once
  // stage k's scores have consumed the previous ones) arrive while stage k
  // finishes
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): setup loads landed
  int ph_cur = nst > 0 ? stage_page(0) : -1;
  if (nst > 0) {
    issue_v(0, ph_cur, sV0, sDoc0);
    load_k(0, ph_cur);
  }
  for (int k = 0; k < nst; k += 2) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    int ph_nxt = k + 1 < nst ? stage_page(k + 1) : -1;
    if (k + 1 < nst) issue_v(k + 1, ph_nxt, sV1, sDoc1);
    f32x16 s[2];
    if (ph_cur >= 0) scores(s);
    if (k + 1 < nst) load_k(k + 1, ph_nxt);
    compute(k, ph_cur, s, sV0, sDoc0);
    if (k + 1 >= nst) break;
    ph_cur = ph_nxt;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    ph_nxt = k + 2 < nst ? stage_page(k + 2) : -1;
    if (k + 2 < nst) issue_v(k + 2, ph_nxt, sV0, sDoc0);
    if (ph_cur >= 0) scores(s);
    if (k + 2 < nst) load_k(k + 2, ph_nxt);
    compute(k + 1, ph_cur, s, sV1, sDoc1);
    ph_cur = ph_nxt;
  }

  // epilogue
  const float l_tot = row_pair_sum(l_run + l_run2);
  if (!h_ok) return;
  const int64_t row = static_cast<int64_t>(b) * p.H + h;
  if (p.nsplit > 1) {
    const int64_t prow = static_cast<int64_t>(c) * p.B * p.H + row;
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
    return;
  }
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  __bf16* op = static_cast<__bf16*>(p.o) + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v4 = {oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv,
                        oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv};
      *reinterpret_cast<bf16x4*>(op + dt * 32 + 8 * q4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
    }
  if (g == 0 && p.lse)
    p.lse[row] = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : FA_NEG_INF;
}

}  // namespace fa
