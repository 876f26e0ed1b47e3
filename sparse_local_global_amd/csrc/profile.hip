// Per-kernel HIP-event timing for measurement (pack3d_profile_*).
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace pack3d {
namespace {

struct Pending {
  std::string name;
  hipEvent_t start, stop;
};

struct Totals {
  std::string name;
  int32_t launches = 0;
  double ms = 0.0;
};

std::mutex g_mu;
bool g_enabled = false;
thread_local int g_off = 0;  // ProfileOff scopes alive on this thread
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::vector<Totals> g_totals;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfileOff::ProfileOff() { ++g_off; }
ProfileOff::~ProfileOff() { --g_off; }

ProfileScope::ProfileScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  if (g_off) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled) return;
  Pending p;
  p.name = name;
  p.start = take_event();
  p.stop = take_event();
  if (!p.start || !p.stop) return;
  hipEventRecord(p.start, s);
  g_pending.push_back(p);
  slot = (int)g_pending.size() - 1;
}

ProfileScope::~ProfileScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot < (int)g_pending.size()) hipEventRecord(g_pending[slot].stop, stream);
}

}  // namespace pack3d

using namespace pack3d;

extern "C" pack3d_status pack3d_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_enabled = enable != 0;
  return PACK3D_OK;
}

extern "C" void pack3d_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    hipEventSynchronize(p.stop);
    g_free.push_back(p.start);
    g_free.push_back(p.stop);
  }
  g_pending.clear();
  g_totals.clear();
}

extern "C" int32_t pack3d_profile_read(char* names, size_t names_bytes, int32_t* launches, double* total_ms,
                                       int32_t max_kernels) {
  std::lock_guard<std::mutex> lk(g_mu);
  int32_t rc = 0;
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      rc = -1;
    } else {
      Totals* t = nullptr;
      for (auto& x : g_totals)
        if (x.name == p.name) t = &x;
      if (!t) {
        g_totals.push_back(Totals{p.name, 0, 0.0});
        t = &g_totals.back();
      }
      t->launches += 1;
      t->ms += ms;
    }
    g_free.push_back(p.start);
    g_free.push_back(p.stop);
  }
  g_pending.clear();
  if (rc < 0) return -1;
  int32_t n = 0;
  size_t off = 0;
  for (auto& t : g_totals) {
    if (n >= max_kernels) break;
    const size_t len = t.name.size() < 47 ? t.name.size() : 47;
    if (!names || off + len + 1 > names_bytes) break;
    std::memcpy(names + off, t.name.data(), len);
    names[off + len] = '\0';
    off += len + 1;
    if (launches) launches[n] = t.launches;
    if (total_ms) total_ms[n] = t.ms;
    ++n;
  }
  return n;
}
