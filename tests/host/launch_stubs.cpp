// Host-only stand-ins for the kernel launchers (test infrastructure): the C
// entry points' argument checks, planners and host arithmetic are built with
// the host sanitizers and linked against these instead of the HIP kernels.
// Each stand-in counts its calls and touches nothing; the workspace sizes are
// simple positive formulas.
#include <hip/hip_runtime_api.h>

#include "mla_internal.h"

int g_launches = 0;

namespace mla {

static hipError_t counted() {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_kv_append(void*, int, int, const int*, int, int, const void*, const void*,
                            const int*, const int*, int, const RopeFreq&, hipStream_t) {
  return counted();
}
hipError_t launch_kv_append_fp8(void*, float*, int, int, const int*, int, int, const void*,
                                const void*, const int*, const int*, int, const RopeFreq&,
                                hipStream_t) {
  return counted();
}
hipError_t launch_absorb_q(const void*, const void*, const void*, const int*, int, int, int,
                           const RopeFreq&, void*, hipStream_t) {
  return counted();
}
hipError_t launch_append_absorb(void*, int, int, const int*, int, int, const void*, const void*,
                                const int*, const int*, int, const void*, const void*,
                                const void*, const int*, int, int, const RopeFreq&, void*,
                                hipStream_t) {
  return counted();
}
hipError_t launch_decode(const void*, const void*, int, const int*, int, const int*, int, int, int,
                         int, float, int, const int*, int, const int*, int, float*, float*, float*,
                         float*, int, hipStream_t) {
  return counted();
}
hipError_t launch_decode_h64(const void*, const void*, int, const int*, int, const int*, int, int,
                             int, float, int, const int*, int, const int*, int, float*, float*,
                             float*, float*, int, hipStream_t) {
  return counted();
}
hipError_t launch_decode_fp8(const void*, const void*, const float*, int, const int*, int,
                             const int*, int, int, int, float, int, const int*, int, const int*,
                             int, float*, float*, float*, float*, int, hipStream_t) {
  return counted();
}
hipError_t launch_combine(const float*, const float*, int, int, int, int, float*, float*,
                          hipStream_t) {
  return counted();
}
hipError_t launch_combine_planned(const float*, const float*, const int*, int, int, float*, float*,
                                  hipStream_t) {
  return counted();
}
hipError_t launch_out_proj(const float*, const void*, int, int, int, float*, hipStream_t) {
  return counted();
}
hipError_t launch_out_proj_planned(float*, const float*, const float*, const int*, int,
                                   const void*, int, int, int, float*, float*, hipStream_t) {
  return counted();
}
long kv_produce_workspace(int T, int d_model) { return 4L * T * 576 + d_model; }
long q_produce_workspace(int T, int d_model, int d_cq, int) { return 4L * T * d_cq + d_model; }
hipError_t launch_kv_produce(const void*, const void*, const float*, const void*, int, int, int,
                             float, const RopeFreq&, void*, int, const int*, int, int, const int*,
                             const int*, void*, hipStream_t) {
  return counted();
}
hipError_t launch_q_produce(const void*, const void*, const float*, const void*, const void*, int,
                            int, int, int, int, float, void*, void*, void*, hipStream_t) {
  return counted();
}
hipError_t launch_q_produce_direct(const void*, const void*, const void*, int, int, int, int,
                                   void*, void*, hipStream_t) {
  return counted();
}
long o_proj_workspace(int T, int n_h, int d_model, int) { return 2L * T * n_h * 128 + d_model; }
hipError_t launch_o_proj(const float*, const void*, int, int, int, int, void*, void*,
                         hipStream_t) {
  return counted();
}
long prefill_mha_workspace(int max_len, int n_h) { return 6L * n_h * 128 * (max_len + 256); }
hipError_t launch_prefill_mha(const void*, const void*, const int*, const void*, const void*,
                              const void*, int, const int*, int, const int*, int, int, int, float,
                              const RopeFreq&, float*, float*, void*, hipStream_t) {
  return counted();
}

}  // namespace mla
