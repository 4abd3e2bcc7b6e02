// Internal helpers shared by the library's translation units: the thread-local
// error text, argument checks and HIP error mapping.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/fsa.h"

namespace fsa {

// Records a message for fsa_last_error() and returns the status.
fsa_status fail(fsa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread's error text (called on entry of every API function).
void clear_error();
// Maps the last launch error to FSA_E_HIP (or FSA_OK).
fsa_status check_launch(const char *what);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace fsa

#define FSA_REQUIRE(cond, status, ...)                 \
  do {                                                 \
    if (!(cond)) return ::fsa::fail(status, __VA_ARGS__); \
  } while (0)
