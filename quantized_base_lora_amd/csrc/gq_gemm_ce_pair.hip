// LM-head backward launches that pair the gradient tiles of one vocabulary
// chunk with the dh tiles of the previous chunk (ce_bwd_dh_kernel in
// gq_gemm_impl.h), one instantiation per quant type.
#include "gq_gemm_impl.h"

namespace gq {
hipError_t launch_ce_bwd_dh_q(int qtype, const GemmArgs& ce, const GemmArgs& dh, hipStream_t st) {
  const int nce = ce.mtiles * ce.ntiles, ndh = dh.mtiles * dh.ntiles;
  if (nce <= 0 || ndh <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nce + ndh));
  switch (qtype) {
    case QT_Q8_0: mmq_launch(ce_bwd_dh_kernel<QT_Q8_0>, grid, dim3(NTHR), st, ce, dh, nce); break;
    case QT_Q4_0: mmq_launch(ce_bwd_dh_kernel<QT_Q4_0>, grid, dim3(NTHR), st, ce, dh, nce); break;
    case QT_Q2_DM: mmq_launch(ce_bwd_dh_kernel<QT_Q2_DM>, grid, dim3(NTHR), st, ce, dh, nce); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace gq
