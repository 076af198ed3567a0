// MFMA GEMM instantiations: Q4_0 blocks, forward (NT) epilogues.
#include "gq_gemm_impl.h"
#include "gq_skinny_impl.h"
#include "gq_wide_impl.h"

namespace gq {
hipError_t launch_gemm_q4_0_nt(int epi, int tilecfg, const GemmArgs& a, hipStream_t st) {
  switch (epi) {
    case EPI_LIN: return launch_q<QT_Q4_0, EPI_LIN>(tilecfg, a, st);
    case EPI_SWIGLU: return launch_q<QT_Q4_0, EPI_SWIGLU>(tilecfg, a, st);
    case EPI_CE_FWD: return launch_q<QT_Q4_0, EPI_CE_FWD>(tilecfg, a, st);
    case EPI_CE_BWD: return launch_q<QT_Q4_0, EPI_CE_BWD>(tilecfg, a, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace gq
