// dsa_host.hpp -- the thread-local error message behind dsa_last_error().
#pragma once

namespace dsa_host {
// Stores the formatted message for dsa_last_error() and returns `code`.
int set_error(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
}  // namespace dsa_host
