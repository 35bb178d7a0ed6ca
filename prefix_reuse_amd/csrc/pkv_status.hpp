// Host-only declaration shared by the sources that are not HIP: they report
// their status through the same thread-local message as the kernel entry
// points (pkv_last_error()).
#pragma once

namespace pkv {
int record_status(int code, const char* msg);
}  // namespace pkv
