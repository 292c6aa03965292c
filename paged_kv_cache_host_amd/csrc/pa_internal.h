// Declarations shared by the host translation units of libpa.
#pragma once

#include "pa.h"

namespace pa {

// Record a printf-style message as the calling thread's last error and
// return `st`.
pa_status fail(pa_status st, const char* fmt, ...);

}  // namespace pa
