// bf16 attention backward instances for head dimension 64: the dQ kernel and
// the dK / dV kernel, after the preparation kernels (bwd_prepare.hip).
#include "bwd_bf16.hpp"

namespace fa {

int launch_bwd_bf16_d64(const BwdLaunch& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FwdLaunch& f = p.f;
  const int q_items = f.B * f.H * f.nqb;
  const int kv_items = f.B * f.H_kv * f.nkvb;
  const dim3 qgrid(static_cast<unsigned>((q_items + 7) / 8 * 8));  // whole XCD rounds
  const dim3 kgrid(static_cast<unsigned>((kv_items + 7) / 8 * 8));
  switch (f.block_m * 4 + f.score_kind) {
#define FA_CASE(BLK, SC)                                                                     \
  case BLK * 4 + SC:                                                                         \
    if (q_items > 0) hipLaunchKernelGGL((bwd_dq_kernel<64, BLK, SC>), qgrid, dim3(BLK * 2), 0, s, p); \
    if (kv_items > 0)                                                                        \
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, BLK, SC>), kgrid, dim3(BLK * 2), 0, s, p);      \
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
