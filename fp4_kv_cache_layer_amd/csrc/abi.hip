// Library-wide entry points of the CSA2 C ABI: version, device check, status text, the
// per-thread record of the last HIP error, and the device status word.
#include <atomic>
#include <mutex>
#include <string.h>

#include "device.h"

static thread_local char g_last_error[256] = {0};

// The device status word: a kernel that meets a condition it cannot express in its outputs
// (a bounded wait that gave up) stores a nonzero CSA2_STATUS_* code into it.  It sits in
// pinned, mapped, coherent host memory, so every call reads it on the host without a
// device synchronisation; csa2_init allocates it once per process (4 bytes; every device
// maps pinned host memory at the same address).  Kernels store into it with plain
// system-scope stores, never read-modify-write, so no atomics cross the host link.
static uint32_t* g_status_host = nullptr;
static uint32_t* g_status_dev = nullptr;
static std::once_flag g_status_once;
static int g_status_rc = CSA2_OK;
static std::atomic<int> g_wait_limit{1 << 22};

uint32_t* csa2_status_word() { return g_status_dev; }
int csa2_wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }

static const char* device_status_text(uint32_t code) {
  switch (code) {
    case CSA2_STATUS_ATTN_WAIT:
      return "an attention kernel gave up waiting for its partner wave; that call's output and lse are invalid";
    default: return "a kernel reported an unknown device status";
  }
}

int csa2_take_device_status() {
  if (!g_status_host) return CSA2_OK;
  const uint32_t code = __atomic_load_n(g_status_host, __ATOMIC_ACQUIRE);
  if (code == 0) return CSA2_OK;
  __atomic_store_n(g_status_host, 0u, __ATOMIC_RELEASE);
  strncpy(g_last_error, device_status_text(code), sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
  return CSA2_ERR_DEVICE;
}

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
    case CSA2_ERR_DEVICE: return "a kernel of an earlier call reported a device-side failure (see csa2_last_error)";
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
  {   // the no-allocation attention entry point's static scratch on this device
    int src = CSA2_OK;
    if (!csa2_attn_scratch(&src)) return src != CSA2_OK ? src : CSA2_ERR_HIP;
  }
  std::call_once(g_status_once, [] {
    void* h = nullptr;
    int rc = csa2_record_hip_error(
        hipHostMalloc(&h, 64, hipHostMallocPortable | hipHostMallocMapped | hipHostMallocCoherent));
    void* d = nullptr;
    if (rc == CSA2_OK) rc = csa2_record_hip_error(hipHostGetDevicePointer(&d, h, 0));
    if (rc == CSA2_OK) {
      *static_cast<volatile uint32_t*>(h) = 0u;
      g_status_host = static_cast<uint32_t*>(h);
      g_status_dev = static_cast<uint32_t*>(d);
    }
    g_status_rc = rc;
  });
  return g_status_rc;
}

extern "C" uint32_t csa2_device_status(int clear) {
  if (!g_status_host) return 0u;
  const uint32_t code = __atomic_load_n(g_status_host, __ATOMIC_ACQUIRE);
  if (clear) __atomic_store_n(g_status_host, 0u, __ATOMIC_RELEASE);
  return code;
}

extern "C" int csa2_debug_set_wait_limit(int polls) {
  const int prev = g_wait_limit.load();
  g_wait_limit.store(polls < 0 ? (1 << 22) : polls);
  return prev;
}
