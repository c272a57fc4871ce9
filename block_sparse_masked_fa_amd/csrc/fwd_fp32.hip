// fp32 attention forward instances (head dimensions 64 and 128).
#include "fwd_fp32.hpp"

namespace fa {

int launch_fwd_fp32(const FwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(p.B * p.H * p.nqb));
  const int key = (p.D * 1000 + p.block_m) * 4 + p.score_kind;
  switch (key) {
#define FA_CASE(D, BLK, SC)                                                    \
  case (D * 1000 + BLK) * 4 + SC:                                              \
    hipLaunchKernelGGL((fwd_fp32_kernel<D, BLK, SC>), grid, dim3(BLK * 2), 0,  \
                       s, p);                                                  \
    break;
    FA_CASE(64, 64, FA_SCORE_NONE)
    FA_CASE(64, 64, FA_SCORE_SOFTCAP)
    FA_CASE(64, 64, FA_SCORE_ALIBI)
    FA_CASE(64, 128, FA_SCORE_NONE)
    FA_CASE(64, 128, FA_SCORE_SOFTCAP)
    FA_CASE(64, 128, FA_SCORE_ALIBI)
    FA_CASE(128, 64, FA_SCORE_NONE)
    FA_CASE(128, 64, FA_SCORE_SOFTCAP)
    FA_CASE(128, 64, FA_SCORE_ALIBI)
    FA_CASE(128, 128, FA_SCORE_NONE)
    FA_CASE(128, 128, FA_SCORE_SOFTCAP)
    FA_CASE(128, 128, FA_SCORE_ALIBI)
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
