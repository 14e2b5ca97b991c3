// Internal to libsv: error reporting and call tags shared by the library's source files. Not
// installed.
#ifndef SV_INTERNAL_H_
#define SV_INTERNAL_H_

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

// Records msg as the message sv_last_error() returns on this thread and returns status.
__attribute__((visibility("hidden"))) int sv_internal_fail(int status, const char* msg);
// Clears this thread's message (every entry point starts with it).
__attribute__((visibility("hidden"))) void sv_internal_clear_error();

// Call tags. Work-groups of one launch hand values to each other as 64-bit words whose upper
// half is a tag of the call; a reader takes a word for this call's exactly when the tag matches.
// Tags come from one process-wide 64-bit counter: a call takes `step` consecutive values, and
// their low 32 bits, [*tag, *tag + step), are its tags (never 0, never wrapping inside a call).
// When the counter's low 32 bits wrap, old words could carry tags handed out again, so the first
// call on a workspace in each wrap period (and the first call on a workspace the library has not
// seen) enqueues a zero fill of its `bytes` bytes on stream s before the launch. Returns SV_OK, or
// SV_ERR_HIP when the fill could not be launched.
__attribute__((visibility("hidden"))) int sv_internal_call_tags(uint32_t step, void* ws,
                                                                size_t bytes, hipStream_t s,
                                                                uint32_t* tag);

// Enqueues a zero fill of [ws, ws + bytes) on stream s (a kernel, no memset: it may be captured
// into a HIP graph). Returns SV_OK, or SV_ERR_HIP when the fill could not be launched.
__attribute__((visibility("hidden"))) int sv_internal_zero_fill(void* ws, size_t bytes,
                                                                hipStream_t s);

// Records that the library is about to leave untagged words in ws (per-position Markov launches,
// top-K tables): the next call that takes tags on ws zero-fills it first.
__attribute__((visibility("hidden"))) void sv_internal_untagged_use(void* ws);

#endif  // SV_INTERNAL_H_
