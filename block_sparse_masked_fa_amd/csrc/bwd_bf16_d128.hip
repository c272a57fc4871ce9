// bf16 attention backward instances for head dimension 128: the dQ kernel and
// the dK / dV kernel, after the preparation kernels (bwd_prepare.hip).
#include "bwd_bf16.hpp"

namespace fa {

int launch_bwd_bf16_d128(const BwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FwdLaunch& f = p.f;
  const int q_items = f.B * f.H * f.nqb * f.nsplit;
  const int kv_items = f.B * f.H_kv * f.nkvb * p.kv_splits;
  const dim3 qgrid(static_cast<unsigned>((q_items + 7) / 8 * 8));  // whole XCD rounds
  const dim3 kgrid(static_cast<unsigned>((kv_items + 7) / 8 * 8));
  switch ((f.block_m * 1000 + f.block_n) * 4 + f.score_kind) {
#define FA_CASE(BQ, BK, SC)                                                                  \
  case (BQ * 1000 + BK) * 4 + SC:                                                            \
    if (q_items > 0)                                                                         \
      hipLaunchKernelGGL((bwd_dq_kernel<128, BQ, BK, SC>), qgrid, dim3(BQ * 2), 0, s, p);     \
    if (kv_items > 0)                                                                        \
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, BQ, BK, SC>), kgrid, dim3(BK * 2), 0, s, p);   \
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
