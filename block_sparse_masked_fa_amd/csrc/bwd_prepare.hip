// Backward preparation, before the gradient kernels:
//   * the block lists transposed: for each key block n, the query blocks m
//     whose row lists name n (partial and full apart), in ascending m. The
//     dK / dV kernel walks them. Built from the forward's lists (whatever
//     their origin) through a dense byte matrix of tile states: cleared,
//     scattered per query-block row, then compacted per key-block column
//     with wavefront ballots and prefix counts.
// and the split backward's last step: the parts' fp32 gradient sums added in
// part order, scaled and rounded to bf16.
#include <hip/hip_runtime.h>

#include "fwd_common.hpp"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void clear_kernel(unsigned char* s, int64_t n) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < n;
       t += static_cast<int64_t>(gridDim.x) * kThreads)
    s[t] = 0;
}

// one workgroup per (b, h, m) row of the forward lists
__global__ __launch_bounds__(kThreads) void scatter_kernel(const BwdLaunch p) {
  const FwdLaunch& f = p.f;
  const int64_t row = blockIdx.x;
  const int nkvb = f.nkvb;
  unsigned char* st = p.states + row * nkvb;
  const int np = min(max(f.num[row], 0), nkvb);
  const int32_t* pl = f.idx + row * nkvb;
  for (int t = threadIdx.x; t < np; t += kThreads) {
    const int n = pl[t];
    if (static_cast<unsigned>(n) < static_cast<unsigned>(nkvb)) st[n] = 1;
  }
  __syncthreads();  // a block named in both lists ends up full, whichever thread wrote first
  if (f.fnum) {
    const int nf = min(max(f.fnum[row], 0), nkvb);
    const int32_t* fl = f.fidx + row * nkvb;
    for (int t = threadIdx.x; t < nf; t += kThreads) {
      const int n = fl[t];
      if (static_cast<unsigned>(n) < static_cast<unsigned>(nkvb)) st[n] = 2;
    }
  }
}

// exclusive prefix count of `flag` over the workgroup; *total: the count
__device__ int wg_prefix(bool flag, int* wave_counts, int* total) {
  const int wave = threadIdx.x >> 6;
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(flag);
  const int lane_prefix = __builtin_amdgcn_mbcnt_hi(
      static_cast<unsigned>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u));
  if ((threadIdx.x & 63) == 0) wave_counts[wave] = __builtin_popcountll(mask);
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += (w < wave) ? wave_counts[w] : 0;
    sum += wave_counts[w];
  }
  __syncthreads();
  *total = sum;
  return before + lane_prefix;
}

// one workgroup per (b, h, n) column
__global__ __launch_bounds__(kThreads) void transpose_kernel(const BwdLaunch p) {
  __shared__ int wave_counts[kWaves];
  const FwdLaunch& f = p.f;
  const int nqb = f.nqb, nkvb = f.nkvb;
  const int64_t col = blockIdx.x;  // (b, h) * nkvb + n
  const int64_t bh = col / nkvb;
  const int n = static_cast<int>(col % nkvb);
  const unsigned char* st = p.states + bh * nqb * nkvb + n;
  int32_t* qi = p.qidx + col * nqb;
  int32_t* fqi = p.fqidx ? p.fqidx + col * nqb : nullptr;
  int run_p = 0, run_f = 0;
  for (int base = 0; base < nqb; base += kThreads) {
    const int m = base + threadIdx.x;
    const int s = m < nqb ? st[static_cast<int64_t>(m) * nkvb] : 0;
    int cp, cf;
    const int pp = run_p + wg_prefix(s == 1, wave_counts, &cp);
    const int pf = run_f + wg_prefix(s == 2, wave_counts, &cf);
    if (s == 1) qi[pp] = m;
    if (s == 2) fqi[pf] = m;
    run_p += cp;
    run_f += cf;
  }
  if (threadIdx.x == 0) {
    p.qnum[col] = run_p;
    if (p.fqnum) p.fqnum[col] = run_f;
  }
}

__global__ __launch_bounds__(kThreads) void zero16_kernel(uint4* dst, int64_t n16) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < n16;
       t += static_cast<int64_t>(gridDim.x) * kThreads)
    dst[t] = uint4{0u, 0u, 0u, 0u};
}

// out[e] = bf16(mul * (parts[0][e] + parts[1][e] + ...)), parts added in
// index order; 8 elements per thread and iteration, two segments (dK and
// dV: same size, own scale) per launch.
struct ReduceSeg {
  const float* parts;
  __bf16* out;
  float mul;
};

__global__ __launch_bounds__(kThreads) void reduce_parts_kernel(ReduceSeg s0, ReduceSeg s1,
                                                                int nseg, int64_t n8,
                                                                int64_t part_elems, int nsplit) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int sg = 0; sg < nseg; ++sg) {
    const ReduceSeg sd = sg == 0 ? s0 : s1;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < n8; t += stride) {
      const float* src = sd.parts + t * 8;
      f32x4 a = *reinterpret_cast<const f32x4*>(src);
      f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      for (int c = 1; c < nsplit; ++c) {
        src += part_elems;
        a += *reinterpret_cast<const f32x4*>(src);
        b += *reinterpret_cast<const f32x4*>(src + 4);
      }
      const f32x8 r = {a[0] * sd.mul, a[1] * sd.mul, a[2] * sd.mul, a[3] * sd.mul,
                       b[0] * sd.mul, b[1] * sd.mul, b[2] * sd.mul, b[3] * sd.mul};
      *reinterpret_cast<bf16x8*>(sd.out + t * 8) = __builtin_convertvector(r, bf16x8);
    }
  }
}

}  // namespace

int launch_reduce_parts(const float* parts0, void* out0, float mul0, const float* parts1,
                        void* out1, float mul1, uint64_t elems, int nsplit, void* stream) {
  const int64_t n8 = static_cast<int64_t>(elems / 8);
  if (n8 == 0) return hipSuccess;
  const ReduceSeg s0{parts0, static_cast<__bf16*>(out0), mul0};
  const ReduceSeg s1{parts1, static_cast<__bf16*>(out1), mul1};
  const int64_t g = (n8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(reduce_parts_kernel, dim3(static_cast<unsigned>(g < 4096 ? g : 4096)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(stream), s0, s1,
                     parts1 ? 2 : 1, n8, static_cast<int64_t>(elems), nsplit);
  return hipGetLastError();
}

int launch_zero_fill(void* dst, uint64_t bytes, void* stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t g = (n16 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(zero16_kernel, dim3(static_cast<unsigned>(g < 8192 ? g : 8192)), dim3(kThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

int launch_bwd_prepare(const BwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FwdLaunch& f = p.f;
  const dim3 blk(kThreads);
  const int64_t lrows = static_cast<int64_t>(f.Bm) * f.Hm * f.nqb;
  const int64_t cells = lrows * f.nkvb;
  if (cells > 0) {
    const int64_t g = (cells + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>(g < 4096 ? g : 4096)), blk, 0, s,
                       p.states, cells);
    hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(lrows)), blk, 0, s, p);
  }
  // one workgroup per key-block column; with no query blocks it only
  // writes zero counts
  const int64_t cols = static_cast<int64_t>(f.Bm) * f.Hm * f.nkvb;
  if (cols > 0)
    hipLaunchKernelGGL(transpose_kernel, dim3(static_cast<unsigned>(cols)), blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
