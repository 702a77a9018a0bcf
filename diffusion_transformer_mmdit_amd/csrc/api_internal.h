// Library-internal entry points shared by the C ABI translation units.
#pragma once
#include <stddef.h>

#include "../../include/mmdit.h"

namespace mmdit {

// Sets the calling thread's mmdit_last_error() text and returns `code`.
int fail(int code, const char* fmt, ...);

// mmdit_step_ex on a workspace of ws_bytes at ws (checked against
// mmdit_step_workspace before any launch).
int step_impl(const mmdit_config* cfg, const mmdit_model_w* w, void* x_packed, void* v_out, const void* txt_emb,
              const void* y, const int32_t* ids, double sigma, double sigma_next, const mmdit_step_opts* opts,
              void* ws, size_t ws_bytes, void* hip_stream);

}  // namespace mmdit
