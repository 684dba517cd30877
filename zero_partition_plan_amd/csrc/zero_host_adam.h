// Shared between the host update (zero_host_adam.cpp) and the offloaded step (zero_offload.cpp).
#pragma once

#include "zero_internal.h"

namespace zero {

// Argument checks of the host update; need_grad: grad must be non-NULL when n > 0.
zero_status check_host_args(const char* fn, bool need_grad, const float* grad, uint64_t n,
                            float* master, float* m, float* v, const zero_adam_hparams* hp,
                            void* out, int32_t out_dtype, zero_adam_scalars* k);

// The update of [0, n) on host arrays with the given constants, split over `threads` threads.
zero_status host_step(const float* grad, uint64_t n, float grad_scale, float* master, float* m,
                      float* v, const zero_adam_scalars& k, bool l2, void* out, int out_dtype,
                      uint32_t threads);

}  // namespace zero
