// Per-thread status text shared by the library's host-side entry points.
#pragma once

#include "pensieve.h"

namespace pk {

// Record `msg` as the calling thread's last error and return `s`.
pensieve_status set_error(pensieve_status s, const char* msg);
// Clear the calling thread's last error and return PENSIEVE_OK.
pensieve_status clear_error();

}  // namespace pk
