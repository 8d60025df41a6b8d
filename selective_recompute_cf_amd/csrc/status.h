// Error state shared by the host-side translation units of libcf (internal).
#pragma once
#include "cf.h"

namespace cf {
// Clears the thread-local text that cf_last_error() returns.
void clear_error();
// Stores msg as the thread-local error text and returns s.
cf_status set_error(cf_status s, const char* msg);
}  // namespace cf
