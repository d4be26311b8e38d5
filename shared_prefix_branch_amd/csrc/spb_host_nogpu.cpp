// spb_host_nogpu.cpp -- kernel launchers for the host-only sanitizer build of
// libspb (spb_host.cpp built by g++ with AddressSanitizer and
// UndefinedBehaviorSanitizer, no GPU code).  That build checks the planner,
// the plan accessors and every host-side validation; it runs no kernel.  Each
// launcher here refuses the launch with hipErrorNoBinaryForGpu, so a call that
// passes validation fails loudly with SPB_ERR_HIP instead of computing
// anything.  Never linked into the GPU library.
#include "spb_launch.h"

#include <hip/hip_runtime_api.h>

namespace spb {

namespace {
constexpr int kNoKernels = (int)hipErrorNoBinaryForGpu;
}

int launch_attention(const AttnLaunch &, void *) { return kNoKernels; }
int launch_score(const ScoreLaunch &, void *) { return kNoKernels; }
int launch_score_batch(const ScoreBatchLaunch &, void *) { return kNoKernels; }
int launch_rmsnorm(const NormLaunch &, void *) { return kNoKernels; }
int launch_linear(const LinearLaunch &, void *) { return kNoKernels; }
int launch_quantize_e4m3(const QuantLaunch &, void *) { return kNoKernels; }
int launch_gather_rows(const GatherLaunch &, void *) { return kNoKernels; }
int launch_topk_lse(const TopkLaunch &, void *) { return kNoKernels; }
int launch_decode_attention(const DecodeAttnLaunch &, void *) { return kNoKernels; }
int launch_beam_step(const BeamLaunch &, void *) { return kNoKernels; }
int score_scratch(void **) { return kNoKernels; }
int launch_mfma_calibration(float *, int, int, int, void *) { return kNoKernels; }
const char *hip_error_string(int err) {
  return err == kNoKernels ? "this host-only build holds no GPU kernels" : hipGetErrorString((hipError_t)err);
}

}  // namespace spb
