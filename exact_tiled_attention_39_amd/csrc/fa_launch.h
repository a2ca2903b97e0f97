// Internal interface between the C-ABI entry points (fa_api.cpp) and the HIP kernels
// (fa_fwd.hip, fa_bwd.hip). Not installed; callers use include/fa.h.
#pragma once

#include "fa.h"

namespace fa {

// Enqueues the forward kernel for arguments that fa_check_args already accepted.
// On a HIP error returns FA_ERR_LAUNCH and sets *hip_error to the HIP error text.
fa_status launch_forward(const fa_fwd_params& p, void* stream, const char** hip_error);

// Enqueues the three backward kernels for arguments that fa_bwd_check_args already accepted.
fa_status launch_backward(const fa_bwd_params& p, void* stream, const char** hip_error);

}  // namespace fa
