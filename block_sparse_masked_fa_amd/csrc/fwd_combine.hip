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

// One wavefront per row. Lane r < nsplit (at most 64) fetches part r's
// (m_r, l_r), so the maximum and the weights w_r = 2^(m_r - m) come from
// wave reductions; then lane L accumulates elements [L * E, L * E + E) of D
// over the parts, with the parts' loads issued four at a time.
template <int D>
__global__ __launch_bounds__(64) void split_combine_kernel(const CombineLaunch p) {
  constexpr int E = D / 64;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int ns = p.nsplit;
  float mr = FA_NEG_INF, lr = 0.0f;
  if (lane < ns) {
    const int64_t pr = lane * p.rows + row;
    mr = p.part_ml[2 * pr];
    lr = p.part_ml[2 * pr + 1];
  }
  float m = mr;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  const float wr = mr == FA_NEG_INF ? 0.0f : exp2_hw(mr - m);
  float l = wr * lr;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  const float* base = p.part_o + row * D + lane * E;
  const int64_t step = p.rows * D;  // between parts
  int r = 0;
  for (; r + 4 <= ns; r += 4) {
    float v[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = base[(r + u) * step + e];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = __shfl(wr, r + u);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, v[u][e], acc[e]);
    }
  }
  for (; r < ns; ++r) {
    const float w = __shfl(wr, r);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, base[r * step + e], acc[e]);
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
  const dim3 grid(static_cast<unsigned>(p.rows));
  if (p.D == 64)
    hipLaunchKernelGGL((split_combine_kernel<64>), grid, dim3(64), 0, s, p);
  else if (p.D == 128)
    hipLaunchKernelGGL((split_combine_kernel<128>), grid, dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
