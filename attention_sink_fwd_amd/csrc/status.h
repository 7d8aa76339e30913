// Host-side error reporting shared by the C-ABI entry points.
#pragma once

namespace sinkattn {

// Thread-local error text for sink_attn_last_error(): fail() formats it and
// returns `status`; clear_error() empties it at the start of an entry point.
int fail(int status, const char* fmt, ...);
void clear_error();

}  // namespace sinkattn
