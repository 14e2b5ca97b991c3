// Internal to libsv: error reporting shared by the library's source files. Not installed.
#ifndef SV_INTERNAL_H_
#define SV_INTERNAL_H_

// Records msg as the message sv_last_error() returns on this thread and returns status.
__attribute__((visibility("hidden"))) int sv_internal_fail(int status, const char* msg);
// Clears this thread's message (every entry point starts with it).
__attribute__((visibility("hidden"))) void sv_internal_clear_error();

#endif  // SV_INTERNAL_H_
