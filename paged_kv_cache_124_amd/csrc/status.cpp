// Status strings and ABI version of libpa.so.
#include "pa.h"

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_NO_FREE_BLOCKS: return "no free blocks in the pool";
    case PA_ERR_EXISTS: return "sequence already exists";
    case PA_ERR_NOT_FOUND: return "sequence not found";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int pa_version(void) { return 2; }
