// timing.cpp - optional per-kernel timing with HIP events (aq_kernel_timing / aq_kernel_times).
//
// While enabled, each kernel the library launches is bracketed by two HIP events recorded on the
// launch stream; aq_kernel_times() waits for the recorded events and reports, per kernel name,
// the number of launches and their summed duration.  Disabled (the default), launches carry no
// extra work.
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "timing.hpp"

namespace aq {
namespace {

struct Pending {
  const char *name;
  hipEvent_t start, stop;
};

struct Totals {
  long count = 0;
  double ms = 0.0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::map<std::string, Totals> g_totals;

}  // namespace

bool timing_on() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on;
}

void timing_begin(hipEvent_t *start, hipStream_t stream) {
  *start = nullptr;
  if (hipEventCreate(start) != hipSuccess) {
    *start = nullptr;
    return;
  }
  hipEventRecord(*start, stream);
}

void timing_end(const char *name, hipEvent_t start, hipStream_t stream) {
  if (!start) return;
  hipEvent_t stop;
  if (hipEventCreate(&stop) != hipSuccess) {
    hipEventDestroy(start);
    return;
  }
  hipEventRecord(stop, stream);
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({name, start, stop});
}

}  // namespace aq

extern "C" {

int aq_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(aq::g_mu);
  aq::g_on = enable != 0;
  return 0;
}

int aq_kernel_times(char *buf, size_t len, int reset) {
  std::vector<aq::Pending> todo;
  {
    std::lock_guard<std::mutex> lk(aq::g_mu);
    todo.swap(aq::g_pending);
  }
  std::map<std::string, aq::Totals> add;
  int rc = 0;
  for (auto &p : todo) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
      rc = -3;
    auto &t = add[p.name];
    t.count += 1;
    t.ms += ms;
    hipEventDestroy(p.start);
    hipEventDestroy(p.stop);
  }
  std::string out;
  {
    std::lock_guard<std::mutex> lk(aq::g_mu);
    for (auto &kv : add) {
      aq::g_totals[kv.first].count += kv.second.count;
      aq::g_totals[kv.first].ms += kv.second.ms;
    }
    char line[256];
    for (auto &kv : aq::g_totals) {
      snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.count, kv.second.ms);
      out += line;
    }
    if (reset) aq::g_totals.clear();
  }
  if (buf && len) {
    strncpy(buf, out.c_str(), len - 1);
    buf[len - 1] = '\0';
  }
  return rc ? rc : (int)out.size();
}

}  // extern "C"
