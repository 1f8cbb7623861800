// vs_status_string / vs_version.
#include "common.h"

extern "C" const char* vs_status_string(int status) {
  switch (status) {
    case VS_OK: return "VS_OK";
    case VS_ERR_INVALID_ARG: return "VS_ERR_INVALID_ARG: null pointer, negative size or bad mode";
    case VS_ERR_UNSUPPORTED: return "VS_ERR_UNSUPPORTED: head dim, cluster count, size or alignment not supported";
    case VS_ERR_WORKSPACE: return "VS_ERR_WORKSPACE: workspace missing or too small";
    case VS_ERR_HIP: return "VS_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown vsmooth status";
  }
}

extern "C" const char* vs_version(void) { return "0.1.0"; }
