// Internal entry points shared by the C-ABI sources (api.cpp, noalloc.hip).
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "swa_sdpa.h"

namespace swa {

// Workspace bytes a backward plan needs.
size_t bwd_plan_workspace_bytes(const sdpa_bwd_plan_t* plan);

// The backward's validation and launch sequence (sdpa_bwd_run_events);
// check_ws_ptr: ask the runtime whether `ws` is device memory of the
// current device.
sdpa_status bwd_run(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* t, void* ws, size_t ws_bytes,
                    hipStream_t stream, hipEvent_t main_start, hipEvent_t main_stop, bool check_ws_ptr);

// Sets the thread-local message sdpa_last_error() returns; returns st.
sdpa_status set_error(sdpa_status st, const char* msg);

}  // namespace swa
