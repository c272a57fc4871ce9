// Device helpers shared by the attention kernels: vector types, the built-in
// mask_mods and score_mods, and tanh written from its definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flexattn.h"
#include "internal.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const int32_t const_i32;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
#define FA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float exp2_hw(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// tanh x = 1 - 2 / (e^{2x} + 1), evaluated on |x| and given the sign of x.
// e^{2|x|} overflows to +inf for large |x|, giving exactly 1. Absolute error
// is a few float ulps of 1 (the cancellation near 0 is absolute, not
// relative), far below what the score tolerance needs.
__device__ __forceinline__ float tanh_def(float x) {
  const float ax = __builtin_fabsf(x);
  const float e = exp2_hw(ax * (2.0f * kLog2e));
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return __builtin_copysignf(t, x);
}

// Score modification in the log2 domain: the kernels keep scores multiplied
// by log2(e) so the softmax uses exp2. For raw = q.k:
//   NONE     s2 = raw * scale * log2e
//   ALIBI    s2 = (raw * scale - slope_h * (i - j)) * log2e
//   SOFTCAP  s2 = cap * tanh(raw * scale / cap) * log2e
struct ScoreConsts {
  float c;              // scale * log2e
  float slope2;         // slope_h * log2e
  float c_over_slope2;  // scale / slope_h
  float cap_in;         // scale / cap
  float cap_out;        // cap * log2e
};

template <class Params>
__device__ __forceinline__ ScoreConsts make_score_consts(const Params& p, int h) {
  ScoreConsts k;
  k.c = p.scale * kLog2e;
  // slope_h = 2^(-8 (h + 1) / H)
  const float slope = exp2_hw(-8.0f * static_cast<float>(h + 1) / static_cast<float>(p.H));
  k.slope2 = slope * kLog2e;
  k.c_over_slope2 = p.scale / slope;
  k.cap_in = p.score_kind == FA_SCORE_SOFTCAP ? p.scale / p.softcap : 0.0f;
  k.cap_out = p.score_kind == FA_SCORE_SOFTCAP ? p.softcap * kLog2e : 0.0f;
  return k;
}

template <int SCORE>
__device__ __forceinline__ float score2(float raw, const ScoreConsts& k,
                                        float i_minus_j) {
  if constexpr (SCORE == FA_SCORE_ALIBI) {
    return __builtin_fmaf(-k.slope2, i_minus_j, raw * k.c);
  } else if constexpr (SCORE == FA_SCORE_SOFTCAP) {
    return k.cap_out * tanh_def(raw * k.cap_in);
  } else {
    return raw * k.c;
  }
}

// mask_mod built-ins (True = allowed). `dj` is doc_id[j] for the document
// mask, `di` is doc_id[i].
template <int KIND>
__device__ __forceinline__ bool mask_ok(int i, int j, int window, int di,
                                        int dj) {
  if constexpr (KIND == FA_MASK_CAUSAL) {
    return i >= j;
  } else if constexpr (KIND == FA_MASK_SLIDING_WINDOW) {
    const int d = i - j;
    return (d >= 0) & (d < window);
  } else if constexpr (KIND == FA_MASK_LOCAL_WINDOW) {
    const int d = i - j;
    return (d < window) & (-d < window);
  } else if constexpr (KIND == FA_MASK_DOCUMENT) {
    return (i >= j) & (di == dj);
  } else {
    return true;
  }
}

// Work item of one workgroup: query block m of head (b, h). Workgroups are
// numbered head-major; inside a head the query blocks run from the last
// (heaviest under causal masks) to the first.
struct WorkItem {
  int b, h, m;
  int c = 0;  // split-KV part
};

__device__ __forceinline__ WorkItem work_item(const FwdLaunch& p) {
  const int wg = blockIdx.x;
  WorkItem w;
  w.m = p.nqb - 1 - (wg % p.nqb);
  const int bh = wg / p.nqb;
  w.h = bh % p.H;
  w.b = bh / p.H;
  return w;
}

}  // namespace fa
