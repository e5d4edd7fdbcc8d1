// Thread-local last-error message shared by every translation unit of librf.
#pragma once

namespace rf {
void set_last_error(const char* msg);
}  // namespace rf
