// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <stdint.h>

#include "../../include/blink.h"

namespace blink {

// Records `code` and a printf-style message for the calling thread; returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's message; returns BLINK_OK.
int ok();
// Compute units of the current device, read from the runtime once per device and kept (a
// property of the hardware, not of any call); a call then costs one hipGetDevice. On failure
// records "<who>: no device" and returns BLINK_E_DEVICE.
int device_cus(int &cus, const char *who);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace blink
