// Status strings and ABI version of libdsv.
#include "dsv.h"

extern "C" const char *dsv_status_string(dsv_status s) {
  switch (s) {
    case DSV_OK: return "ok";
    case DSV_ERR_INVALID_ARG: return "invalid argument";
    case DSV_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSV_ERR_WORKSPACE: return "workspace missing or too small";
    case DSV_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

extern "C" int dsv_abi_version(void) { return DSV_ABI_VERSION; }

extern "C" size_t dsv_attn_args_size(void) { return sizeof(dsv_attn_args); }
