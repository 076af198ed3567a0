// Dispatch of the MFMA GEMM template (gq_gemm_impl.h) by quant type and
// epilogue; the instantiations live in one translation unit per (type, mode)
// so they compile in parallel.
#include "gq_dev.h"
#include "gq_internal.h"

namespace gq {
hipError_t launch_gemm_q8_0_nt(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_q8_0_nn(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_q4_0_nt(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_q4_0_nn(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_q2_dm_nt(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_q2_dm_nn(int epi, int tilecfg, const GemmArgs& a, hipStream_t st);
hipError_t launch_ce_bwd_dh_q(int qtype, const GemmArgs& ce, const GemmArgs& dh, hipStream_t st);

namespace {
// optional timing events of every MMQ launch of this thread (mmq_launch)
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

hipError_t dispatch(int qtype, int epi, int tilecfg, const GemmArgs& a, hipStream_t st) {
  const bool nn = epi >= EPI_LIN_BWD;
  switch (qtype) {
    case QT_Q8_0: return nn ? launch_gemm_q8_0_nn(epi, tilecfg, a, st) : launch_gemm_q8_0_nt(epi, tilecfg, a, st);
    case QT_Q4_0: return nn ? launch_gemm_q4_0_nn(epi, tilecfg, a, st) : launch_gemm_q4_0_nt(epi, tilecfg, a, st);
    case QT_Q2_DM: return nn ? launch_gemm_q2_dm_nn(epi, tilecfg, a, st) : launch_gemm_q2_dm_nt(epi, tilecfg, a, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

void set_profile_events(hipEvent_t start, hipEvent_t stop) {
  g_prof_start = start;
  g_prof_stop = stop;
}

hipEvent_t profile_event(int stop) { return stop ? g_prof_stop : g_prof_start; }

hipError_t launch_gemm(int qtype, int epi, int tilecfg, const GemmArgs& a, hipStream_t st) {
  if ((int64_t)a.mtiles * a.ntiles == 0) return hipSuccess;
  return dispatch(qtype, epi, tilecfg, a, st);
}

hipError_t launch_ce_bwd_dh(int qtype, const GemmArgs& ce, const GemmArgs& dh, hipStream_t st) {
  return launch_ce_bwd_dh_q(qtype, ce, dh, st);
}
}  // namespace gq
