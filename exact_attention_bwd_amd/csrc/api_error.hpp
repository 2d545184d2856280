// The thread-local status message behind attn_last_error(), for entry points
// defined outside attn_api.hip.
#pragma once

#include "../../include/attn_mi355x.h"

namespace attn {

// Sets the calling thread's attn_last_error() message (printf format) and
// returns `st`.
attn_status report(attn_status st, const char* fmt, ...);

}  // namespace attn
