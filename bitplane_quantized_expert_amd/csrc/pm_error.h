// The last-error channel of libpm (pm_last_error), shared by its host files.
#pragma once

#include "../../include/pm.h"

namespace pm {
// Records the formatted message for pm_last_error() and returns st.
pm_status failf(pm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
}  // namespace pm
