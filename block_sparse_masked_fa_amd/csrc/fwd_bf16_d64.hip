// bf16 attention forward instances for head dimension 64.
#include "fwd_bf16.hpp"
#include "fwd_bf16_v2.hpp"

namespace fa {

int launch_fwd_bf16_d64(const FwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(p.B * p.H * p.nqb));
  const int key = p.block * 4 + p.score_kind;
  switch (key) {
#define FA_CASE(BLK, SC)                                                      \
  case BLK * 4 + SC:                                                          \
    hipLaunchKernelGGL((fwd_bf16_kernel<64, BLK, SC>), grid, dim3(BLK * 2), 0, \
                       s, p);                                                 \
    break;
    FA_CASE(64, FA_SCORE_NONE)
    FA_CASE(64, FA_SCORE_SOFTCAP)
    FA_CASE(64, FA_SCORE_ALIBI)
#define FA_CASE2(SC)                                                          \
  case 128 * 4 + SC:                                                          \
    hipLaunchKernelGGL((fwd_bf16_v2_kernel<64, SC>), grid, dim3(512), 0, s, p); \
    break;
    FA_CASE2(FA_SCORE_NONE)
    FA_CASE2(FA_SCORE_SOFTCAP)
    FA_CASE2(FA_SCORE_ALIBI)
#undef FA_CASE2
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
