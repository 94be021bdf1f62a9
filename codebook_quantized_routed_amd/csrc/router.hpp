// Launchers of the router projection kernels (k_router.hip).
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

hipError_t launch_router(const float *x, const float *wr, const float *wsg, int T, int H, int E, float *logits,
                         float *sw, hipStream_t s);
hipError_t launch_shared_weight(const float *sw, int T, int kprime, float *w, hipStream_t s);

}  // namespace moe
