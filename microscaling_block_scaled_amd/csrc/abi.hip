// abi.hip -- status strings and the device-support check of libmxfp8.
#include <atomic>
#include <cstring>

#include "mx_common.hpp"

namespace {
// Per-device answer of the architecture check, filled on first use and never
// changed afterwards (0 = not yet known, 1 = gfx950, 2 = other), and the
// device's compute-unit count, filled with it.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];

const char* kReasonOk = "gfx950 device: MXFP8 quantize and scaled-MFMA GEMM available";
const char* kReasonArch = "libmxfp8 is built for gfx950 (MI355X) only; this device is a different architecture";
const char* kReasonNoDevice = "no HIP device with this index";

int arch_state(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 2;
  int s = g_arch_state[dev].load(std::memory_order_acquire);
  if (s != 0) return s;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 2;
  s = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  g_cu_count[dev].store(p.multiProcessorCount, std::memory_order_relaxed);
  g_arch_state[dev].store(s, std::memory_order_release);
  return s;
}
}  // namespace

namespace mx_host {
mx_status_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MX_ERR_DEVICE;
  return arch_state(dev) == 1 ? MX_OK : MX_ERR_DEVICE;
}
int cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || arch_state(dev) == 2) return 0;
  return g_cu_count[dev].load(std::memory_order_relaxed);
}
}  // namespace mx_host

extern "C" const char* mx_status_string(mx_status_t status) {
  switch (status) {
    case MX_OK: return "MX_OK: success";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: bad size or pitch (blocked dimensions must be multiples of 32)";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: base address or pitch is not 16-byte aligned";
    case MX_ERR_FORMAT: return "MX_ERR_FORMAT: unknown element format or data type";
    case MX_ERR_DEVICE: return "MX_ERR_DEVICE: the current device is not gfx950";
    case MX_ERR_HIP: return "MX_ERR_HIP: the HIP runtime reported an error at launch";
    default: return "unknown mx_status_t";
  }
}

extern "C" mx_status_t mx_query_support(int device, const char** reason) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) {
    if (reason) *reason = kReasonNoDevice;
    return MX_ERR_DEVICE;
  }
  const bool ok = arch_state(device) == 1;
  if (reason) *reason = ok ? kReasonOk : kReasonArch;
  return ok ? MX_OK : MX_ERR_DEVICE;
}
