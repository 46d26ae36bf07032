// Internal entry points of the C ABI shared between fa_api.cpp and the
// translation units that add calls on top of it.  Nothing here is exported.
#pragma once
#include "../../include/flash_attn.h"

namespace fa {

// Supplies the backward workspace once every argument has been validated:
// given the bytes the call needs and its stream, sets *ws and *bytes and
// returns FA_OK, or returns a status (with flash_attn_last_error() set).
typedef fa_status (*WorkspaceFn)(const char* fn, size_t need, hipStream_t stream, void** ws, size_t* bytes);

// flash_attn_bwd with the workspace taken from get_ws instead of the
// caller's arguments (get_ws runs only for non-empty, valid problems).
fa_status bwd_dense_with(const char* fn, int B, int H, int N, int d, fa_dtype dtype, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse, float scale, int causal,
                         void* dq, void* dk, void* dv, WorkspaceFn get_ws, hipStream_t stream);

// Records a thread-local error message and returns s.
fa_status fail_status(fa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace fa
