// bf16 attention forward instances for head dimension 64.
#include "fwd_bf16.hpp"

namespace fa {

int launch_fwd_bf16_d64(const FwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int items = p.B * p.H * p.nqb * p.nsplit;
  const dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));  // whole XCD rounds
  const int key = (p.block_m * 1000 + p.block_n) * 4 + p.score_kind;
  switch (key) {
#define FA_CASE(BQ, BK, SC)                                                      \
  case (BQ * 1000 + BK) * 4 + SC:                                                \
    hipLaunchKernelGGL((fwd_bf16_kernel<64, BQ, BK, SC>), grid, dim3(BQ * 2), 0, \
                       s, p);                                                    \
    break;
#define FA_CASES(BQ, BK)           \
  FA_CASE(BQ, BK, FA_SCORE_NONE)    \
  FA_CASE(BQ, BK, FA_SCORE_SOFTCAP) \
  FA_CASE(BQ, BK, FA_SCORE_ALIBI)
    FA_CASES(64, 64)
    FA_CASES(64, 128)
    FA_CASES(128, 64)
    FA_CASES(128, 128)
#undef FA_CASES
#undef FA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
