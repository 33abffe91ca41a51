// pa_error.h -- the per-thread message behind pa_last_error() (internal).
#pragma once

namespace pa {

// Records the formatted message and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns PA_OK.
int ok();
const char* last_error();

}  // namespace pa
