// Status records of the contexts.  Each context owns one record of
// kStatusWords 32-bit words (layout in kernels.h) in a file-scope device array,
// so creating a context allocates no device memory.  Each device holds its own
// copy of the array; its address is looked up once per device with
// hipGetSymbolAddress (the array's name in host code is not a device address).
#include "kernels.h"

#include <bitset>
#include <mutex>

namespace clha {

static __device__ __align__(256) int g_status_records[kMaxContexts * kStatusWords];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
int* g_base[kMaxDevices] = {};
std::bitset<kMaxContexts> g_used[kMaxDevices];
}  // namespace

int* status_acquire(int device, int* slot) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_base[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_status_records)) != hipSuccess || !p) return nullptr;
    g_base[device] = static_cast<int*>(p);
  }
  for (int s = 0; s < kMaxContexts; ++s) {
    if (g_used[device][s]) continue;
    int* rec = g_base[device] + (size_t)s * kStatusWords;
    if (hipMemset(rec, 0, kStatusWords * sizeof(int)) != hipSuccess) return nullptr;
    g_used[device][s] = true;
    *slot = s;
    return rec;
  }
  return nullptr;
}

void status_release(int device, int slot) {
  if (device < 0 || device >= kMaxDevices || slot < 0 || slot >= kMaxContexts) return;
  std::lock_guard<std::mutex> lock(g_mutex);
  g_used[device][slot] = false;
}

}  // namespace clha
