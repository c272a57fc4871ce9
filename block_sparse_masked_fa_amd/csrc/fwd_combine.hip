// Split-KV merge: the partial results of the parts of a row's key-block
// list are combined exactly. Part r covers a set K_r of keys, disjoint from
// the others, and holds m_r = max over K_r of the log2-domain scores,
// l_r = sum_{K_r} 2^(s - m_r) and A_r = sum_{K_r} 2^(s - m_r) v. With
// m = max_r m_r and w_r = 2^(m_r - m):
//   O = sum_r w_r A_r / sum_r w_r l_r,   LSE = (m + log2 sum_r w_r l_r) ln 2,
// the softmax over the union of the K_r (the same sums regrouped). A part
// with no allowed key has m_r = -inf and contributes nothing.
#include <hip/hip_runtime.h>

#include "fwd_common.hpp"

namespace fa {
namespace {

// One wavefront per row; lane L holds elements [L * E, L * E + E) of D.
template <int D>
__global__ __launch_bounds__(256) void split_combine_kernel(const CombineLaunch p) {
  constexpr int E = D / 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int lane = threadIdx.x & 63;
  float m = FA_NEG_INF;
  for (int r = 0; r < p.nsplit; ++r) m = __builtin_fmaxf(m, p.part_ml[2 * (r * p.rows + row)]);
  float l = 0.0f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int r = 0; r < p.nsplit; ++r) {
    const int64_t pr = r * p.rows + row;
    const float mr = p.part_ml[2 * pr];
    const float wr = mr == FA_NEG_INF ? 0.0f : exp2_hw(mr - m);
    l = __builtin_fmaf(wr, p.part_ml[2 * pr + 1], l);
    const float* po = p.part_o + pr * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(wr, po[e], acc[e]);
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  __bf16* op = static_cast<__bf16*>(p.o) + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) op[e] = static_cast<__bf16>(acc[e] * inv);
  if (lane == 0 && p.lse)
    p.lse[row] = l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : FA_NEG_INF;
}

}  // namespace

int launch_split_combine(const CombineLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>((p.rows + 3) / 4));
  if (p.D == 64)
    hipLaunchKernelGGL((split_combine_kernel<64>), grid, dim3(256), 0, s, p);
  else if (p.D == 128)
    hipLaunchKernelGGL((split_combine_kernel<128>), grid, dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
