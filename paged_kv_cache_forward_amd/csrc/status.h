// Status plumbing shared by every translation unit of libpagedattn (host only).
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pagedattn.h"

namespace pa {

// Records a formatted message for pa_last_error() and returns the status.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// True when PA_CHECK=1 is set in the environment (read on every call).
bool check_mode();

}  // namespace pa
