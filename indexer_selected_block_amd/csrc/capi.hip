// Library-wide entry points of the C ABI: version and status text.
#include "isb_host.h"

extern "C" int isb_version(void) { return 200; }  // 0.2.0: the cache writer, query step and candidate merge

extern "C" const char* isb_strerror(int status) {
  switch (status) {
    case ISB_OK: return "ok";
    case ISB_E_INVALID_ARG: return "invalid argument (null pointer or non-positive size)";
    case ISB_E_UNSUPPORTED_DTYPE: return "dtype not supported for this argument";
    case ISB_E_SHAPE: return "shape relation violated";
    case ISB_E_WORKSPACE: return "workspace smaller than isb_sparse_pa_workspace_bytes";
    case ISB_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
