// Internal interface between the C-ABI entry points (fa_api.cpp, fa_plan.cpp) and the HIP
// kernels (fa_fwd.hip, fa_bwd.hip, ...). Not installed; callers use include/fa.h. Everything
// declared here is host code; fa_api.cpp and fa_plan.cpp build with a plain C++ compiler.
#pragma once

#include <cstdint>

#include "fa.h"

namespace fa {

// Enqueues the forward kernel for arguments that fa_check_args already accepted.
// On a HIP error returns FA_ERR_LAUNCH and sets *hip_error to the HIP error text.
fa_status launch_forward(const fa_fwd_params& p, void* stream, const char** hip_error);

// Enqueues the FP8 (E4M3) forward kernel for arguments that fa_check_args accepted.
fa_status launch_forward_fp8(const fa_fwd_params& p, void* stream, const char** hip_error);

// Enqueues the RoPE pass that writes the rotated keys to p.k_rot (p.rope_cos set).
fa_status launch_rope_keys(const fa_fwd_params& p, void* stream, const char** hip_error);

// Split-KV geometry shared by the planner (fa_plan.cpp) and the kernels (fa_splitkv.hip).
constexpr int kSplitTileKeys = 32;   // keys per K/V tile
constexpr int kSplitBlockRows = 32;  // packed query rows per workgroup

// Work decomposition of the split-KV forward for arguments that fa_check_args accepted.
struct SplitPlan {
  int32_t splits = 1;           // key ranges per (sequence, kv head, row block)
  int64_t rowblocks = 0;        // 32-row blocks of packed query rows per (sequence, kv head)
  int64_t items = 0;            // splits * heads_kv * (batch or sequences)
  int64_t grid = 0;             // workgroups of the split kernel (items padded to 8, x rowblocks)
  int64_t rows_total = 0;       // batch * heads_q * seqlen
  uint64_t workspace_bytes = 0; // partial outputs and log-sum-exps (0 with one split)
};

// num_splits in [0, FA_MAX_SPLITS]; 0 picks a count from the shapes.
SplitPlan plan_splitkv(const fa_fwd_params& p, int32_t num_splits);

// Enqueues the split kernel and, with more than one split, the merge kernel.
fa_status launch_forward_splitkv(const fa_fwd_params& p, const SplitPlan& plan, void* workspace,
                                 void* stream, const char** hip_error);

// Device address of the current device's static split-KV scratch (FA_NOALLOC_SCRATCH_BYTES),
// looked up once per device; NULL (and *hip_error set) on a HIP error.
void* noalloc_scratch(const char** hip_error);

// Enqueues the three backward kernels for arguments that fa_bwd_check_args already accepted.
fa_status launch_backward(const fa_bwd_params& p, void* stream, const char** hip_error);

}  // namespace fa
