// errors.hpp -- the thread-local error message behind gdn_last_error(), shared
// by the library's HIP and host-only translation units.  Internal.
#pragma once

#include "gdn_slot.h"

namespace gdn {
// Record a message (printf format) for gdn_last_error() and return `s`.
gdn_status set_error(gdn_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return GDN_OK.
gdn_status clear_error();
}  // namespace gdn
