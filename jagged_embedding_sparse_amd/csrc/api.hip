// Error strings and version of the C ABI declared in fs_sparse.h.
#include "common.hpp"

extern "C" const char* fs_strerror(int code) {
  switch (code) {
    case FS_OK: return "ok";
    case FS_ERR_INVALID_ARG: return "invalid argument";
    case FS_ERR_WORKSPACE: return "workspace missing or too small";
    case FS_ERR_HIP: return "HIP launch failed";
    case FS_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case FS_ERR_TOO_LARGE: return "sizes need more than the fixed scratch of an allocation-free call";
  }
  return "unknown error";
}

extern "C" int fs_version(void) { return 1; }
