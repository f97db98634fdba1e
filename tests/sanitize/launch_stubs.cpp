// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// the C-ABI front end (api.cpp) makes, so that its argument validation can
// be built with host sanitizers and driven without a GPU.  Every launcher
// reports success and records that it was reached.
#include <hip/hip_runtime.h>

#include "../../autoregressive_video_diffusion_amd/csrc/crattn_internal.h"

int g_launches = 0;

namespace crattn {
hipError_t launch_rope_table(const RopeTableArgs &, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_rope_append(const RopeAppendArgs &, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_attn(const AttnArgs &, const AttnPlan &, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_qkv_rope(const QkvArgs &, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_hsa_pool(const HsaPoolArgs &, int, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_hsa_select(const HsaSelectArgs &, int, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_svg2_kmeans(const KmArgs &, int, int, bool, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_svg2_kmeans2(const KmArgs &, const KmArgs &, int, int, bool, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_svg2_plan(const SvgPlanArgs &, int, hipStream_t) { return ++g_launches, hipSuccess; }
static char fake_scratch[256];
void *attn_scratch(hipError_t *err) { *err = hipSuccess; return fake_scratch; }
}  // namespace crattn

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }
