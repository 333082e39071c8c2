// Error reporting shared by the library's host sources (not part of the C ABI).
#pragma once

namespace q8rt {
// Record `msg` as the calling thread's last error (qwen3_last_error) and
// return `code`.
int set_error(int code, const char* msg);
}  // namespace q8rt
