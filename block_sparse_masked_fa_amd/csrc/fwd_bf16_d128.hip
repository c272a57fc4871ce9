// bf16 attention forward instances for head dimension 128.
#include "fwd_bf16.hpp"

namespace fa {

int launch_fwd_bf16_d128(const FwdLaunch& p_in, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int items = p_in.B * p_in.H * p_in.nqb * p_in.nsplit;
  unsigned wgs = 0;
  const FwdLaunch p = fwd_schedule(p_in, items, &wgs);
  const dim3 grid(wgs);
  const int doc = p.mask.kind == FA_MASK_DOCUMENT ? 1 : 0;
  const int key = ((p.block_m * 1000 + p.block_n) * 4 + p.score_kind) * 2 + doc;
  switch (key) {
#define FA_CASE(BQ, BK, SC, DOC)                                                       \
  case ((BQ * 1000 + BK) * 4 + SC) * 2 + DOC:                                          \
    hipLaunchKernelGGL((fwd_bf16_kernel<128, BQ, BK, SC, DOC>), grid, dim3(BQ * 2), 0, s, \
                       p);                                                             \
    break;
#define FA_CASES(BQ, BK)                  \
  FA_CASE(BQ, BK, FA_SCORE_NONE, false)    \
  FA_CASE(BQ, BK, FA_SCORE_SOFTCAP, false) \
  FA_CASE(BQ, BK, FA_SCORE_ALIBI, false)   \
  FA_CASE(BQ, BK, FA_SCORE_NONE, true)     \
  FA_CASE(BQ, BK, FA_SCORE_SOFTCAP, true)  \
  FA_CASE(BQ, BK, FA_SCORE_ALIBI, true)
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
