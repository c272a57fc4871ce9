// Masked softmax over materialised scores, bf16 in, bf16 out, fp32 inside:
// the fallback chain "compare, select the minimum, softmax" of the MLX pull
// request "Fuse the causal mask into the SDPA fallback softmax" as one
// kernel. The mask is applied where the scores are read, so neither a
// boolean mask nor a masked copy of the scores is ever written; masked
// entries come out as exact zeros, and keys outside the row's allowed
// interval are not even read.
//
// Rows of up to 32768 keys (masked_softmax_reg_kernel): one workgroup of
// 256 threads per row holds the row's allowed scores in registers (16-byte
// chunks of 8 scores, thread t owning chunks t + 256 u): one read, the
// maximum, one exponential per score and the sum (workgroup reductions),
// then every output chunk written once: exp2(x - m) / l inside the
// interval, zeros elsewhere.
// Longer rows (masked_softmax_kernel): one wavefront per row in two passes
// over memory, an online (max, sum) per lane, then the normalised write; the
// second pass reads the scores again.
//
// Roofline: HBM. Per row: the allowed chunks' scores read once (2 bytes
// each) and the whole row's probabilities written once (2 bytes).
#include <hip/hip_runtime.h>

#include "fwd_common.hpp"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront per row
constexpr int kUnroll = 4;        // chunks in flight per lane

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ void unpack8(const u32x4 w, float* x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t v = w[e];
    x[2 * e] = __builtin_bit_cast(float, v << 16);
    x[2 * e + 1] = __builtin_bit_cast(float, v & 0xffff0000u);
  }
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void masked_softmax_kernel(
    const SoftmaxLaunch p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = row / p.q_len;
  const int i = static_cast<int>(row % p.q_len);
  const int K = p.kv_len;
  const int64_t qi = static_cast<int64_t>(i) + p.q_offset;  // query position
  const int kind = p.mask.kind;
  const int64_t W = p.mask.window;
  // the allowed interval [lo, hi) of key positions
  int64_t lo = 0, hi = K;
  if (kind == FA_MASK_CAUSAL || kind == FA_MASK_DOCUMENT) {
    hi = qi + 1;
  } else if (kind == FA_MASK_SLIDING_WINDOW) {
    lo = qi - W + 1;
    hi = qi + 1;
  } else if (kind == FA_MASK_LOCAL_WINDOW) {
    lo = qi - W + 1;
    hi = qi + W;
  }
  lo = max(lo, static_cast<int64_t>(0));
  hi = min(hi, static_cast<int64_t>(K));
  const int jlo = static_cast<int>(lo);
  const int jhi = static_cast<int>(max(hi, lo));
  const bool doc_mask = kind == FA_MASK_DOCUMENT;
  const int* doc = p.mask.doc_id;
  const int di = doc_mask && jhi > jlo ? doc[qi] : 0;

  const __bf16* src = static_cast<const __bf16*>(p.scores) + bh * p.ss[0] + i * p.ss[1];
  __bf16* dst = static_cast<__bf16*>(p.probs) + row * K;
  const int c_lo = jlo >> 3;              // chunks holding allowed keys
  const int c_hi = (jhi + 7) >> 3;
  const int n_chunks = K >> 3;

  // masked scores (log2 domain) of one chunk
  auto load_chunk = [&](int c, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + c * 8);
    unpack8(w, x);
    int dj[8];
    if (doc_mask) {
      const int4 a = *reinterpret_cast<const int4*>(doc + c * 8);
      const int4 b = *reinterpret_cast<const int4*>(doc + c * 8 + 4);
      dj[0] = a.x; dj[1] = a.y; dj[2] = a.z; dj[3] = a.w;
      dj[4] = b.x; dj[5] = b.y; dj[6] = b.z; dj[7] = b.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = c * 8 + e;
      bool ok = (j >= jlo) & (j < jhi);
      if (doc_mask) ok &= dj[e] == di;
      x[e] = ok ? x[e] * kLog2e : FA_NEG_INF;
    }
  };

  // pass 1: online max and sum per lane, then over the wave. kUnroll
  // chunks per lane per iteration, their loads issued together.
  float m = FA_NEG_INF, l = 0.0f;
  auto absorb = [&](const float* x) {
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = __builtin_fmaxf(cm, x[e]);
    const float mn = __builtin_fmaxf(m, cm);
    if (mn != FA_NEG_INF) {
      float add = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) add += exp2_hw(x[e] - mn);
      l = __builtin_fmaf(l, exp2_hw(m - mn), add);
      m = mn;
    }
  };
  int c = c_lo + lane;
  for (; c + 64 * (kUnroll - 1) < c_hi; c += 64 * kUnroll) {
    float x[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_chunk(c + 64 * u, x[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) absorb(x[u]);
  }
  for (; c < c_hi; c += 64) {
    float x[8];
    load_chunk(c, x);
    absorb(x);
  }
  const float mw = wave_max(m);
  const float lw = wave_sum(m == FA_NEG_INF ? 0.0f : l * exp2_hw(m - mw));
  const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;

  // pass 2: every output chunk written once (zeros outside the interval)
  auto emit = [&](int cc, const float* x) {
    f32x8 pv;
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = exp2_hw(x[e] - mw) * inv;
    *reinterpret_cast<u32x4*>(dst + cc * 8) =
        __builtin_bit_cast(u32x4, __builtin_convertvector(pv, bf16x8));
  };
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int z_end = inv > 0.0f ? c_lo : n_chunks;  // all zeros for an empty row
  for (int cz = lane; cz < z_end; cz += 64) *reinterpret_cast<u32x4*>(dst + cz * 8) = zero;
  if (inv > 0.0f) {
    for (int cz = c_hi + lane; cz < n_chunks; cz += 64)
      *reinterpret_cast<u32x4*>(dst + cz * 8) = zero;
    c = c_lo + lane;
    for (; c + 64 * (kUnroll - 1) < c_hi; c += 64 * kUnroll) {
      float x[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_chunk(c + 64 * u, x[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) emit(c + 64 * u, x[u]);
    }
    for (; c < c_hi; c += 64) {
      float x[8];
      load_chunk(c, x);
      emit(c, x);
    }
  }
}

// Rows of up to kRegMaxKeys keys: one workgroup per row keeps the row's
// allowed scores in registers, so they are read from memory exactly once
// and each exponential is computed once. Thread t holds chunks
// c_lo + t + 256 u.
constexpr int kRegThreads = 256;
constexpr int kRegChunks = 16;  // chunks per thread
constexpr int kRegMaxKeys = kRegThreads * kRegChunks * 8;

__global__ __launch_bounds__(kRegThreads) void masked_softmax_reg_kernel(const SoftmaxLaunch p) {
  __shared__ float red[kRegThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t bh = row / p.q_len;
  const int i = static_cast<int>(row % p.q_len);
  const int K = p.kv_len;
  const int64_t qi = static_cast<int64_t>(i) + p.q_offset;
  const int kind = p.mask.kind;
  const int64_t W = p.mask.window;
  int64_t lo = 0, hi = K;
  if (kind == FA_MASK_CAUSAL || kind == FA_MASK_DOCUMENT) {
    hi = qi + 1;
  } else if (kind == FA_MASK_SLIDING_WINDOW) {
    lo = qi - W + 1;
    hi = qi + 1;
  } else if (kind == FA_MASK_LOCAL_WINDOW) {
    lo = qi - W + 1;
    hi = qi + W;
  }
  lo = max(lo, static_cast<int64_t>(0));
  hi = min(hi, static_cast<int64_t>(K));
  const int jlo = static_cast<int>(lo);
  const int jhi = static_cast<int>(max(hi, lo));
  const bool doc_mask = kind == FA_MASK_DOCUMENT;
  const int* doc = p.mask.doc_id;
  const int di = doc_mask && jhi > jlo ? doc[qi] : 0;
  const __bf16* src = static_cast<const __bf16*>(p.scores) + bh * p.ss[0] + i * p.ss[1];
  __bf16* dst = static_cast<__bf16*>(p.probs) + row * K;
  const int c_lo = jlo >> 3;
  const int c_hi = (jhi + 7) >> 3;
  const int n_chunks = K >> 3;

  // one read of the allowed chunks (all loads issued before any use)
  u32x4 raw[kRegChunks];
#pragma unroll
  for (int u = 0; u < kRegChunks; ++u) {
    const int c = c_lo + tid + kRegThreads * u;
    raw[u] = c < c_hi ? *reinterpret_cast<const u32x4*>(src + c * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float x[kRegChunks][8];
  float m = FA_NEG_INF;
#pragma unroll
  for (int u = 0; u < kRegChunks; ++u) {
    const int c = c_lo + tid + kRegThreads * u;
    unpack8(raw[u], x[u]);
    int dj[8];
    if (doc_mask && c < c_hi) {
      const int4 a = *reinterpret_cast<const int4*>(doc + c * 8);
      const int4 b = *reinterpret_cast<const int4*>(doc + c * 8 + 4);
      dj[0] = a.x; dj[1] = a.y; dj[2] = a.z; dj[3] = a.w;
      dj[4] = b.x; dj[5] = b.y; dj[6] = b.z; dj[7] = b.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = c * 8 + e;
      bool ok = (j >= jlo) & (j < jhi);
      if (doc_mask) ok &= dj[e] == di;
      x[u][e] = ok ? x[u][e] * kLog2e : FA_NEG_INF;
      m = __builtin_fmaxf(m, x[u][e]);
    }
  }
  // row maximum over the workgroup
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRegThreads / 64; ++w) m = __builtin_fmaxf(m, red[w]);
  __syncthreads();
  // exponentials (once) and their sum
  float l = 0.0f;
  const float mu = m == FA_NEG_INF ? 0.0f : m;
#pragma unroll
  for (int u = 0; u < kRegChunks; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[u][e] = exp2_hw(x[u][e] - mu);
      l += x[u][e];
    }
  l = wave_sum(l);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = 0.0f;
#pragma unroll
  for (int w = 0; w < kRegThreads / 64; ++w) l += red[w];
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  // every output chunk once
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int z_end = inv > 0.0f ? c_lo : n_chunks;
  for (int c = tid; c < z_end; c += kRegThreads) *reinterpret_cast<u32x4*>(dst + c * 8) = zero;
  if (inv > 0.0f) {
    for (int c = c_hi + tid; c < n_chunks; c += kRegThreads)
      *reinterpret_cast<u32x4*>(dst + c * 8) = zero;
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
      const int c = c_lo + tid + kRegThreads * u;
      if (c < c_hi) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = x[u][e] * inv;
        *reinterpret_cast<u32x4*>(dst + c * 8) =
            __builtin_bit_cast(u32x4, __builtin_convertvector(pv, bf16x8));
      }
    }
  }
}

}  // namespace

int launch_masked_softmax(const SoftmaxLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.kv_len <= kRegMaxKeys) {
    hipLaunchKernelGGL(masked_softmax_reg_kernel, dim3(static_cast<unsigned>(p.rows)),
                       dim3(kRegThreads), 0, s, p);
  } else {
    const int64_t blocks = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(masked_softmax_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * kRowsPerBlock), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace fa
