// Library-internal pieces of the C ABI shared between its source files.
#pragma once

#include <string>

#include "../../include/dag_attn.h"
#include "plan.hpp"

struct dag_plan {
  dagattn::Plan p;
};

namespace dagattn {

// Record `msg` as the thread's last error and return `code`.
dag_status set_error(dag_status code, const std::string& msg);

// The forward's validation and launches on a caller-provided workspace.  With
// allow_upload false the plan must already be on the current device (uploading
// allocates); otherwise it is uploaded on first use.
dag_status attn_fwd_impl(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k, const void* v,
                         void* o, float* lse, void* o_lo, void* ws, size_t ws_bytes, void* hip_stream,
                         bool allow_upload);

}  // namespace dagattn
