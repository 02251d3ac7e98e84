// Dynamic LDS above the 64 KiB default needs a per-kernel attribute on each
// device.  Setting it is a host call (hipFuncSetAttribute) that would
// otherwise run before every launch; the largest size set so far for each
// (kernel, device) is remembered, and the attribute is raised only when a
// launch needs more.

#include <map>
#include <mutex>
#include <utility>

#include "launch.hpp"

namespace convrot {

hipError_t allow_dynamic_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> raised;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = raised[{fn, dev}];
  if (bytes <= have) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

}  // namespace convrot
