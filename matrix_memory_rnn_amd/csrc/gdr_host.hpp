// Host-side launch helpers shared by the kernel launchers. They keep no state
// between calls: the device is read from the launch stream, and a kernel's
// dynamic-LDS limit is set on every launch (a host call of about a
// microsecond), so launches from several threads or onto several devices need
// no synchronisation.
#pragma once

#include <hip/hip_runtime.h>

namespace gdr {

// The device a launch on `stream` runs on (the calling thread's current device
// for the null stream).
inline int stream_device(void* stream) {
  int dev = 0;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice((hipStream_t)stream, &d) == hipSuccess) return (int)d;
  }
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

// Compute units of the device that `stream` belongs to (256 on MI355X).
inline int stream_cus(void* stream) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, stream_device(stream)) != hipSuccess ||
      n <= 0)
    n = 256;
  return n;
}

// Allows `kern` up to `bytes` of dynamic LDS (needed above 64 KiB).
inline bool allow_lds(const void* kern, int bytes) {
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
}

}  // namespace gdr
