// MFMA GEMM instantiations: Q4_0 blocks, backward (NN) epilogues.
#include "gq_gemm_impl.h"
#include "gq_skinny_impl.h"
#include "gq_wide_nn_impl.h"

namespace gq {
hipError_t launch_gemm_q4_0_nn(int epi, int tilecfg, const GemmArgs& a, hipStream_t st) {
  switch (epi) {
    case EPI_LIN_BWD: return launch_q<QT_Q4_0, EPI_LIN_BWD>(tilecfg, a, st);
    case EPI_DOWN_BWD: return launch_q<QT_Q4_0, EPI_DOWN_BWD>(tilecfg, a, st);
    case EPI_GATEUP_BWD: return launch_q<QT_Q4_0, EPI_GATEUP_BWD>(tilecfg, a, st);
    case EPI_DH_ACC: return launch_q<QT_Q4_0, EPI_DH_ACC>(tilecfg, a, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace gq
