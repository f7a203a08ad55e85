// Library-wide entry points of the CSA2 C ABI: version, device check, status text and
// the per-thread record of the last HIP error.
#include <string.h>

#include "device.h"

static thread_local char g_last_error[256] = {0};

int csa2_record_hip_error(hipError_t e) {
  if (e == hipSuccess) return CSA2_OK;
  const char* s = hipGetErrorString(e);
  strncpy(g_last_error, s ? s : "unknown HIP error", sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
  return CSA2_ERR_HIP;
}

int csa2_check_launch() { return csa2_record_hip_error(hipGetLastError()); }

extern "C" int csa2_version(void) { return 100; }

extern "C" const char* csa2_last_error(void) { return g_last_error; }

extern "C" const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "a size, count or shape argument is out of range";
    case CSA2_ERR_UNSUPPORTED: return "unsupported format, dtype or device";
    case CSA2_ERR_HIP: return "the HIP runtime reported an error";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

extern "C" int csa2_init(void) {
  int dev = 0;
  int rc = csa2_record_hip_error(hipGetDevice(&dev));
  if (rc != CSA2_OK) return rc;
  hipDeviceProp_t prop;
  rc = csa2_record_hip_error(hipGetDeviceProperties(&prop, dev));
  if (rc != CSA2_OK) return rc;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    strncpy(g_last_error, prop.gcnArchName, sizeof(g_last_error) - 1);
    return CSA2_ERR_UNSUPPORTED;
  }
  return CSA2_OK;
}
