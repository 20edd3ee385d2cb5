// Helpers shared by the files that define C ABI entry points.  Not part of
// the C ABI (see include/hisparse.h).
#pragma once

#include "hisparse.h"

namespace hsp {

// Record `fmt` as the calling thread's last error (hisparse_last_error) and
// return `code`.
int set_error(int code, const char* fmt, ...);

// The HIP device a handle was created on (-1 for NULL).
int handle_device(const struct hisparse* h);

// Look up, once per device, the device address of the no-alloc attention's
// scratch array on device `dev` (which must be current).
int noalloc_setup(int dev);

}  // namespace hsp
