// Fused block-sparse attention forward, bf16, 128-row blocks: the gfx950
// pipeline.
//
// Work split. One workgroup per (query block of 128 rows, head); 8 wavefronts.
// Wave w owns query tile qt = w % 4 (32 rows) and key half kh = w / 4 (64 of
// the 128 keys of every key block). Two wavefronts therefore share each SIMD,
// so one's MFMA work overlaps the other's softmax arithmetic. Each wave keeps
// its own online-softmax state (running max m, running sum l, output
// accumulator) over its key half; the two halves are merged once at the end:
// m = max(m0, m1), O = (e^(m0-m) O0 + e^(m1-m) O1) / (e^(m0-m) l0 + e^(m1-m) l1).
//
// Data movement. K and V tiles [128 keys][D] stream HBM -> LDS with
// global_load_lds_dwordx4 (no register staging), double-buffered: the tile of
// the next live block is in flight while the current one is consumed. In LDS a
// tile is row-major with its 16-byte chunks XOR-swizzled per row, so that the
// two read patterns below hit distinct banks:
//   - S^T = K Q^T reads K as the MFMA A operand (ds_read_b128: 16 rows, one
//     chunk each);
//   - O^T += V^T P^T needs V transposed (keys along each lane's k slots):
//     ds_read_b64_tr_b16 delivers it straight from the row-major tile
//     (4 rows x 4 chunks per 32 lanes).
// Q^T stays in registers as the B operand for the whole row; P comes out of the
// S^T accumulator already in B-operand layout (lane = query, slots = keys).
//
// Per live block, per wave: 16 MFMA 32x32x16 for S^T, score_mod on all 64 x 32
// positions, mask_mod on partial blocks only, exp2-based online softmax with a
// single cross-half lane exchange for the row max, 16 MFMA for PV.
#pragma once

#include "fwd_common.hpp"

namespace fa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// XOR swizzle of the 16-byte chunks of LDS row r (see the header comment).
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ i16x4 ds_read_tr(const __bf16* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((const char*)base + byte_off));
}

template <int D, int SCORE>
__global__ __launch_bounds__(512, 1) void fwd_bf16_v2_kernel(const FwdLaunch p) {
  constexpr int BLK = 128;
  constexpr int RB = D * 2;            // bytes per LDS row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int TILE = BLK * D;        // elements per tile
  constexpr int ROUNDS = TILE * 2 / (512 * 16);  // DMA rounds per tile
  constexpr int DK = D / 16;
  constexpr int DT = D / 32;

  __shared__ __attribute__((aligned(1024))) __bf16 sK0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[TILE];
  __shared__ int sDoc0[BLK];
  __shared__ int sDoc1[BLK];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;
  const int qt = wave & 3;
  const int kh = wave >> 2;

  const WorkItem w = work_item(p);
  const int hk = w.h / (p.H / p.H_kv);
  const int i = w.m * BLK + qt * 32 + lq;
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

  const int bb = p.Bm == 1 ? 0 : w.b;
  const int hh = p.Hm == 1 ? 0 : w.h;
  const int64_t lrow = (static_cast<int64_t>(bb) * p.Hm + hh) * p.nqb + w.m;
  const int nkvb = p.nkvb;
  const int nf = p.fnum ? min(max(p.fnum[lrow], 0), nkvb) : 0;
  const int np = min(max(p.num[lrow], 0), nkvb);
  const int32_t* fl = p.fidx ? p.fidx + lrow * nkvb : nullptr;
  const int32_t* pl = p.idx + lrow * nkvb;
  const int total = nf + np;

  const ScoreConsts sc = make_score_consts(p, w.h);

  // ---- per-lane LDS byte offsets (independent of the block)
  // K operand: row kh*64 + jt*32 + lq, chunk 2*dk + g
  int k_off[DK];
  {
    const int r = kh * 64 + lq;
    const int s = kv_swz<D>(r);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) k_off[dk] = r * RB + (((2 * dk + g) ^ s) << 4);
  }
  // V transposed reads: row kh*64 + kk*16 + 8*t2 + 4g + (lane%16)/4,
  // d = dt*32 + 16*((lane/16)%2) + 4*(lane%4)
  int v_off[2][DT];
  {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int r = kh * 64 + 8 * t2 + 4 * g + ((lane & 15) >> 2);
      const int s = kv_swz<D>(r);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        v_off[t2][dt] = r * RB + (((d >> 3) ^ s) << 4) + ((d & 7) << 1);
      }
    }
  }
  // DMA: this lane's row / swizzled chunk inside each 1 KB round segment
  constexpr int RPK = 1024 / RB;  // rows per 1 KB
  int dma_row[ROUNDS], dma_col[ROUNDS];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int r = (rd * 8 + wave) * RPK + lane / CPR;
    dma_row[rd] = r;
    dma_col[rd] = ((lane % CPR) ^ kv_swz<D>(r)) * 8;
  }

  auto block_at = [&](int it) -> int {
    const int n = it < nf ? fl[it] : pl[it - nf];
    return n;
  };
  auto issue = [&](int n, __bf16* sK, __bf16* sV, int* sD, bool want_doc) {
    const int j0 = n * BLK;
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int j = min(j0 + dma_row[rd], kv_len - 1);
      const int seg = (rd * 8 + wave) * 1024;
      __builtin_amdgcn_global_load_lds((gbl_void*)(kp + j * ks2 + dma_col[rd]),
                                       (lds_void*)((char*)sK + seg), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void*)(vp + j * vs2 + dma_col[rd]),
                                       (lds_void*)((char*)sV + seg), 16, 0, 0);
    }
    if (want_doc && wave < 2) {
      const int j = min(j0 + wave * 64 + lane, kv_len - 1);
      __builtin_amdgcn_global_load_lds((gbl_void*)(doc + j),
                                       (lds_void*)(sD + wave * 64), 4, 0, 0);
    }
  };

  float m_run = FA_NEG_INF;
  float l_run = 0.0f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  auto compute = [&](int n, bool masked, const __bf16* sK, const __bf16* sV,
                     const int* sD) {
    const int j0 = n * BLK;
    // ---- S^T for this wave's 64 keys
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(sK) + k_off[dk] + jt * 32 * RB);
        s[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[dk],
                                                        s[jt], 0, 0, 0);
      }
    }
    // ---- score_mod; key of (jt, r) = j0 + kh*64 + jt*32 + 8*(r/4) + 4g + r%4
    const float ibase = static_cast<float>(i - j0 - kh * 64 - 4 * g);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[jt][r] = score2<SCORE>(s[jt][r], sc,
                                 ibase - static_cast<float>(jt * 32 + 8 * (r >> 2) + (r & 3)));
    if (masked) {
      const int jb = j0 + kh * 64 + 4 * g;
#define FA_MASK_LOOP(KIND)                                                       \
  _Pragma("unroll") for (int jt = 0; jt < 2; ++jt)                               \
  _Pragma("unroll") for (int r4 = 0; r4 < 4; ++r4) {                             \
    const int jl = jt * 32 + 8 * r4;                                             \
    int dj4[4] = {0, 0, 0, 0};                                                   \
    if (KIND == FA_MASK_DOCUMENT) {                                              \
      const int4 t = *reinterpret_cast<const int4*>(sD + kh * 64 + 4 * g + jl);  \
      dj4[0] = t.x; dj4[1] = t.y; dj4[2] = t.z; dj4[3] = t.w;                    \
    }                                                                            \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) {                              \
      const int j = jb + jl + c;                                                 \
      const bool ok = (j < kv_len) & mask_ok<KIND>(i, j, window, di, dj4[c]);    \
      s[jt][4 * r4 + c] = ok ? s[jt][4 * r4 + c] : FA_NEG_INF;                   \
    }                                                                            \
  }
      switch (mkind) {
        case FA_MASK_CAUSAL: FA_MASK_LOOP(FA_MASK_CAUSAL) break;
        case FA_MASK_SLIDING_WINDOW: FA_MASK_LOOP(FA_MASK_SLIDING_WINDOW) break;
        case FA_MASK_DOCUMENT: FA_MASK_LOOP(FA_MASK_DOCUMENT) break;
        default: FA_MASK_LOOP(FA_MASK_NONE) break;
      }
#undef FA_MASK_LOOP
    }
    // ---- online softmax over this wave's key half
    float mx = FA_NEG_INF;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[jt][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = __builtin_fmaxf(m_run, mx);
    const float m_use = (m_new == FA_NEG_INF) ? 0.0f : m_new;
    float rs = 0.0f;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_hw(s[jt][r] - m_use);
        s[jt][r] = e;
        rs += e;
      }
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float alpha = exp2_hw(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    l_run += rs;
    m_run = m_new;
    // ---- O^T += V^T P^T over this wave's 64 keys (4 k-steps of 16)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f32x16& src = s[kk >> 1];
      const int h8 = (kk & 1) * 8;
      const f32x8 pf = {src[h8 + 0], src[h8 + 1], src[h8 + 2], src[h8 + 3],
                        src[h8 + 4], src[h8 + 5], src[h8 + 6], src[h8 + 7]};
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 lo = ds_read_tr<D>(sV, v_off[0][dt] + kk * 16 * RB);
        const i16x4 hi = ds_read_tr<D>(sV, v_off[1][dt] + kk * 16 * RB);
        const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                              hi[0], hi[1], hi[2], hi[3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb,
                                                           oacc[dt], 0, 0, 0);
      }
    }
  };

  // ---- main loop, unrolled by two so each LDS buffer is a distinct object
  const bool doc_mask = mkind == FA_MASK_DOCUMENT;
  auto is_masked = [&](int it, int n) { return it >= nf || (n + 1) * BLK > kv_len; };
  int n_cur = -1;
  if (total > 0) {
    n_cur = block_at(0);
    issue(n_cur, sK0, sV0, sDoc0, doc_mask && is_masked(0, n_cur));
  }
  for (int it = 0; it < total; it += 2) {
    // even step: buffer 0
    {
      const int n_next = (it + 1 < total) ? block_at(it + 1) : -1;
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (n_next >= 0) issue(n_next, sK1, sV1, sDoc1, doc_mask && is_masked(it + 1, n_next));
      compute(n_cur, is_masked(it, n_cur), sK0, sV0, sDoc0);
      n_cur = n_next;
    }
    if (it + 1 >= total) break;
    // odd step: buffer 1
    {
      const int n_next = (it + 2 < total) ? block_at(it + 2) : -1;
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
      if (n_next >= 0) issue(n_next, sK0, sV0, sDoc0, doc_mask && is_masked(it + 2, n_next));
      compute(n_cur, is_masked(it + 1, n_cur), sK1, sV1, sDoc1);
      n_cur = n_next;
    }
  }

  // ---- merge the two key halves through LDS (the K/V buffers are free now):
  // running stats first, then the accumulator one 32-wide d tile at a time.
  __syncthreads();
  float* ml = reinterpret_cast<float*>(sV0);  // [4 qt][64 lanes][2]
  float* ox = reinterpret_cast<float*>(sK0);  // [4 qt][64 lanes][16]
  const int slot = qt * 64 + lane;
  if (kh == 1) {
    ml[slot * 2] = m_run;
    ml[slot * 2 + 1] = l_run;
  }
  __syncthreads();
  float m = m_run, a0 = 1.0f, a1 = 0.0f, l_tot = 0.0f;
  if (kh == 0) {
    const float m1 = ml[slot * 2];
    const float l1 = ml[slot * 2 + 1];
    m = __builtin_fmaxf(m_run, m1);
    const float mu = (m == FA_NEG_INF) ? 0.0f : m;
    a0 = exp2_hw(m_run - mu);
    a1 = exp2_hw(m1 - mu);
    const float l_lane = l_run * a0 + l1 * a1;
    l_tot = l_lane + __shfl_xor(l_lane, 32);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) ox[slot * 16 + r] = oacc[dt][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] * a0 + ox[slot * 16 + r] * a1;
    }
    __syncthreads();
  }
  if (kh == 0 && i_ok) {
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
      p.lse[orow] = l_tot > 0.0f ? (m + __builtin_amdgcn_logf(l_tot)) * kLn2 : FA_NEG_INF;
  }
}

}  // namespace fa
