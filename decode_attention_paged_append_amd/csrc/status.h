// status.h -- the thread-local error message shared by the library's
// translation units (internal).
#pragma once

#include <string>

#include "pagedattn.h"

namespace pa {

extern thread_local std::string g_last_error;

// Records a printf-style message for pa_last_error() and returns st.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
