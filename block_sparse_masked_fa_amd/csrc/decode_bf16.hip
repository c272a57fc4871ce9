// Decode-step instances over a paged cache (head dimensions 64 and 128).
#include "decode_bf16.hpp"

namespace fa {

int launch_decode_paged(const DecodeLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.H_kv * p.nsplit));
  switch (p.D * 4 + p.score_kind) {
#define FA_CASE(D, SC)                                                                \
  case D * 4 + SC:                                                                    \
    hipLaunchKernelGGL((decode_paged_kernel<D, SC>), grid, dim3(64), 0, s, p);        \
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
