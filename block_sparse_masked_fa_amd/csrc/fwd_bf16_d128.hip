// bf16 attention forward instances for head dimension 128.
#include "fwd_bf16.hpp"

namespace fa {

int launch_fwd_bf16_d128(const FwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int items = p.B * p.H * p.nqb * p.nsplit;
  const dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));  // whole XCD rounds
  const int key = p.block * 4 + p.score_kind;
  switch (key) {
#define FA_CASE(BLK, SC)                                                       \
  case BLK * 4 + SC:                                                           \
    hipLaunchKernelGGL((fwd_bf16_kernel<128, BLK, SC>), grid, dim3(BLK * 2), \
                       0, s, p);                                               \
    break;
    FA_CASE(64, FA_SCORE_NONE)
    FA_CASE(64, FA_SCORE_SOFTCAP)
    FA_CASE(64, FA_SCORE_ALIBI)
    FA_CASE(128, FA_SCORE_NONE)
    FA_CASE(128, FA_SCORE_SOFTCAP)
    FA_CASE(128, FA_SCORE_ALIBI)
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
