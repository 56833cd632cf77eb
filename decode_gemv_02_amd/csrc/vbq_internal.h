// Declarations shared by the host and device halves of the VBQ library.
#pragma once

#include <cstdint>
#include <new>
#include <stdexcept>

#include "vbq.h"

namespace vbq {

// Record a one-line failure description for vbq_last_error() and return st.
// Never throws (the message goes into a fixed thread-local buffer).
vbq_status fail(vbq_status st, const char *fmt, ...) noexcept __attribute__((format(printf, 2, 3)));
void clear_error() noexcept;

// Runs the body of an extern "C" entry point so that no C++ exception crosses
// the ABI: an allocation failure becomes VBQ_ERR_NOMEM, anything else
// VBQ_ERR_INTERNAL, each with a message for vbq_last_error().
template <class F>
vbq_status guarded(const char *who, F &&body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return fail(VBQ_ERR_NOMEM, "%s: host memory exhausted", who);
    } catch (const std::length_error &) {
        return fail(VBQ_ERR_NOMEM, "%s: a host buffer would exceed its maximum size", who);
    } catch (const std::exception &e) {
        return fail(VBQ_ERR_INTERNAL, "%s: unexpected C++ exception: %s", who, e.what());
    } catch (...) {
        return fail(VBQ_ERR_INTERNAL, "%s: unexpected C++ exception", who);
    }
}

}  // namespace vbq
