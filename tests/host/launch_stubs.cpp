// Host-only stand-ins for the kernel launchers of libfa, so that the library's validation and
// planning layer (fa_api.cpp, fa_plan.cpp) links into a CPU test program that runs under
// AddressSanitizer and UndefinedBehaviorSanitizer. Each stand-in counts its calls, touches no
// memory behind the pointers it is given, and reports success.
#include "fa.h"
#include "fa_launch.h"

int g_stub_launches = 0;

namespace fa {

fa_status launch_forward(const fa_fwd_params&, void*, const char**) {
  ++g_stub_launches;
  return FA_OK;
}

fa_status launch_forward_fp8(const fa_fwd_params&, void*, const char**) {
  ++g_stub_launches;
  return FA_OK;
}

fa_status launch_rope_keys(const fa_fwd_params&, void*, const char**) {
  ++g_stub_launches;
  return FA_OK;
}

fa_status launch_forward_splitkv(const fa_fwd_params&, const SplitPlan&, void*, void*,
                                 const char**) {
  ++g_stub_launches;
  return FA_OK;
}

fa_status launch_backward(const fa_bwd_params&, void*, const char**) {
  ++g_stub_launches;
  return FA_OK;
}

void* noalloc_scratch(const char**) { return reinterpret_cast<void*>(uintptr_t(1) << 20); }

}  // namespace fa
