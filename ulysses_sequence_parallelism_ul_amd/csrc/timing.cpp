// Optional per-kernel timing: hipEvents recorded on each kernel's stream,
// accumulated per kernel name until read.  Off by default; a disabled timer
// costs one branch per launch.
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ul_internal.h"

namespace {

struct Pending {
  std::string name;
  hipEvent_t start, stop;
};

struct Totals {
  double ms = 0.0;
  int64_t launches = 0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::map<std::string, Totals> g_totals;
thread_local std::vector<Pending> t_open;

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

// Fold finished pending events into the totals; wait for them if `wait`.
hipError_t drain(bool wait) {
  hipError_t first = hipSuccess;
  std::vector<Pending> keep;
  for (auto& p : g_pending) {
    if (!wait && hipEventQuery(p.stop) != hipSuccess) {
      keep.push_back(p);
      continue;
    }
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess && first == hipSuccess) first = e;
    Totals& t = g_totals[p.name];
    t.ms += ms;
    t.launches += 1;
    g_free.push_back(p.start);
    g_free.push_back(p.stop);
  }
  g_pending.swap(keep);
  return first;
}

}  // namespace

namespace ul {

bool timing_on() { return g_on; }

void timing_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  Pending p{name, take_event(), take_event()};
  if (p.start) (void)hipEventRecord(p.start, s);
  t_open.push_back(p);
}

void timing_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (t_open.empty()) return;
  Pending p = t_open.back();
  t_open.pop_back();
  if (p.start && p.stop && hipEventRecord(p.stop, s) == hipSuccess) g_pending.push_back(p);
  if (g_pending.size() > 4096) (void)drain(false);
}

}  // namespace ul

extern "C" {

int32_t ul_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  const bool was = g_on;
  g_on = on != 0;
  return was ? 1 : 0;
}

void ul_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  (void)drain(true);
  g_totals.clear();
}

int32_t ul_timing_read(int32_t index, char* name, size_t name_len, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (drain(true) != hipSuccess) return -1;
  if (index < 0) return (int32_t)g_totals.size();
  if (index >= (int32_t)g_totals.size()) return -1;
  auto it = g_totals.begin();
  std::advance(it, index);
  if (name && name_len) {
    strncpy(name, it->first.c_str(), name_len - 1);
    name[name_len - 1] = '\0';
  }
  if (total_ms) *total_ms = it->second.ms;
  if (launches) *launches = it->second.launches;
  return (int32_t)g_totals.size();
}

}  // extern "C"
