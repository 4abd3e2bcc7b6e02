// Thread-local error text and the ABI version query.
#include <cstring>
#include <string>

#include "fsa_internal.h"

namespace {
thread_local std::string g_error;
}

namespace fsa {

fsa_status fail(fsa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

void clear_error() { g_error.clear(); }

fsa_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return FSA_OK;
}

}  // namespace fsa

extern "C" int32_t fsa_abi_version(void) { return FSA_ABI_VERSION; }

extern "C" const char *fsa_last_error(void) { return g_error.c_str(); }
