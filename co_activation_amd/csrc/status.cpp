// Host-side helper of the C ABI.
#include "moe_coact.h"

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_ALIGN: return "row size or pointer alignment not supported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
  }
}
