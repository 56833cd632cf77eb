// Declarations shared by the host and device halves of the VBQ library.
#pragma once

#include <cstdint>

#include "vbq.h"

namespace vbq {

// Record a one-line failure description for vbq_last_error() and return st.
vbq_status fail(vbq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace vbq
