// Per-device launch facts shared by the kernels' launchers.
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "attn_internal.hpp"

namespace attn {

namespace {
struct Entry {
  int dev;
  const void* kernel;
  int block;
  int resident;
};
std::mutex g_mu;
std::vector<Entry> g_cache;  // a handful of (device, kernel) pairs
}  // namespace

hipError_t resident_workgroups(int dev, const void* kernel, int block, int* out) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Entry& e : g_cache)
      if (e.dev == dev && e.kernel == kernel && e.block == block) {
        *out = e.resident;
        return hipSuccess;
      }
  }
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
  if (e != hipSuccess) return e;
  const int resident = cus * per_cu;
  std::lock_guard<std::mutex> lk(g_mu);
  g_cache.push_back(Entry{dev, kernel, block, resident});
  *out = resident;
  return hipSuccess;
}

}  // namespace attn
