// Per-device facts and settings that the launches need and that would
// otherwise cost a host call before every launch, each remembered per
// (kernel, device) behind one mutex:
//  * dynamic LDS above the 64 KiB default needs a per-kernel attribute; the
//    largest size set so far is remembered and the attribute raised only
//    when a launch needs more;
//  * a persistent grid is sized by the device's CU count and by how many
//    workgroups of a kernel fit on one CU.

#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "launch.hpp"

namespace convrot {
namespace {
std::mutex g_mu;
}  // namespace

hipError_t allow_dynamic_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  static std::map<std::pair<const void*, int>, size_t> raised;
  std::lock_guard<std::mutex> lock(g_mu);
  size_t& have = raised[{fn, dev}];
  if (bytes <= have) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

hipError_t resident_grid(const void* fn, int threads, size_t lds, int64_t* wgs) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  static std::map<std::tuple<const void*, int, int, size_t>, int64_t> known;
  std::lock_guard<std::mutex> lock(g_mu);
  const auto key = std::make_tuple(fn, dev, threads, lds);
  auto it = known.find(key);
  if (it != known.end()) {
    *wgs = it->second;
    return hipSuccess;
  }
  int cus = 0, per_cu = 0;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev); e != hipSuccess)
    return e;
  if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds); e != hipSuccess)
    return e;
  *wgs = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  known.emplace(key, *wgs);
  return hipSuccess;
}

}  // namespace convrot
