// pinned_pool.cpp -- see pinned_pool.hpp.
#include "pinned_pool.hpp"

#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

namespace cdma {
namespace {

struct Buffer {
  void* p;
  size_t bytes;
  bool in_use;
};

std::mutex pool_mu;
std::vector<Buffer>& pool() {
  static std::vector<Buffer>* v = new std::vector<Buffer>();  // never destroyed: buffers live until exit
  return *v;
}

}  // namespace

void* pinned_acquire(size_t bytes) {
  std::lock_guard<std::mutex> lock(pool_mu);
  Buffer* best = nullptr;
  for (Buffer& b : pool())
    if (!b.in_use && b.bytes >= bytes && (!best || b.bytes < best->bytes)) best = &b;
  if (best) {
    best->in_use = true;
    return best->p;
  }
  size_t cap = 4096;
  while (cap < bytes) cap *= 2;
  void* p = nullptr;
  if (hipHostMalloc(&p, cap, hipHostMallocPortable) != hipSuccess || !p) return nullptr;
  pool().push_back(Buffer{p, cap, true});
  return p;
}

void pinned_release(void* p) {
  if (!p) return;
  std::lock_guard<std::mutex> lock(pool_mu);
  for (Buffer& b : pool())
    if (b.p == p) b.in_use = false;
}

}  // namespace cdma
