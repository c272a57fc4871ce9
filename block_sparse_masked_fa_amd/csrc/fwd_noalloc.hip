// Split-KV forward without any allocation: fa_flex_attention_fwd_split with
// its partial results kept in a fixed device array of this library instead
// of a caller workspace (for callers that cannot allocate: code under HIP
// graph capture, tight serving loops).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. In
// host code the variable's name is only a host-side stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and that address is what the kernels receive. Calls on one
// GPU share the array: calls in flight at the same time on that GPU race.
// Nothing in it has to start at zero: every part writes each of its rows
// (a part with no keys writes a neutral partial result) before the merge
// reads them.
#include <hip/hip_runtime.h>

#include <atomic>
#include <string>

#include "../../include/flexattn.h"
#include "internal.hpp"
#include "validate.hpp"

namespace {

constexpr uint64_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// device address of `scratch` per device ordinal, 0 until looked up
std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];

fa_status noalloc_finish(int status, const std::string& msg) {
  if (status != FA_OK) fa::record_error(msg);
  return static_cast<fa_status>(status);
}

// The current device's copy of `scratch`; 0 with *err set on failure.
uintptr_t scratch_address(std::string* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return 0;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = "device ordinal " + std::to_string(dev) + " out of range";
    return 0;
  }
  uintptr_t ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    return 0;
  }
  ptr = reinterpret_cast<uintptr_t>(p);
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // same value from any thread
  return ptr;
}

}  // namespace

extern "C" {

fa_status fa_flex_attention_fwd_split_noalloc(
    int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t q_len,
    int32_t kv_len, int32_t D, const void* q, const int64_t q_stride[3],
    const void* k, const int64_t k_stride[3], const void* v,
    const int64_t v_stride[3], float scale, const fa_block_mask* bm,
    const fa_score_mod* score, int32_t num_splits, void* o, float* lse,
    void* stream) {
  std::string msg;
  fa::FwdLaunch p{};
  bool nothing = false;
  int st = fa::check_flex_attention_fwd(dtype, B, H, H_kv, q_len, kv_len, D, q,
                                        q_stride, k, k_stride, v, v_stride,
                                        scale, bm, score, o, lse, &p, &nothing,
                                        &msg);
  if (st != FA_OK) return noalloc_finish(st, msg);
  uint64_t need = 0;
  st = fa::check_split_workspace_bytes(B, H, q_len, D, num_splits, &need, &msg);
  if (st != FA_OK) return noalloc_finish(st, msg);
  if (need > kScratchBytes)
    return noalloc_finish(FA_ERR_INVALID_VALUE,
                          "split-KV partial results need " + std::to_string(need) +
                              " bytes; the static scratch holds " +
                              std::to_string(kScratchBytes) +
                              " (use fa_flex_attention_fwd_split with a workspace)");
  void* ws = nullptr;
  if (num_splits > 1) {
    const uintptr_t ptr = scratch_address(&msg);
    if (!ptr) return noalloc_finish(FA_ERR_HIP, msg);
    ws = reinterpret_cast<void*>(ptr);
  }
  fa::CombineLaunch cl{};
  st = fa::check_split(dtype, num_splits, ws, kScratchBytes, &p, &cl, &msg);
  if (st != FA_OK) return noalloc_finish(st, msg);
  if (nothing) return FA_OK;
  int err;
  if (dtype == FA_FP32)
    err = fa::launch_fwd_fp32(p, stream);
  else if (D == 64)
    err = fa::launch_fwd_bf16_d64(p, stream);
  else
    err = fa::launch_fwd_bf16_d128(p, stream);
  if (err == 0 && p.nsplit > 1) err = fa::launch_split_combine(cl, stream);
  if (err != 0)
    return noalloc_finish(FA_ERR_HIP, std::string("split-KV launch: ") +
                                          hipGetErrorString(static_cast<hipError_t>(err)));
  return FA_OK;
}

}  // extern "C"
