// side_stream.hip - a second stream per device for launch sequences whose steps do not all depend
// on each other: the K/V prepass of the cube-sparse forward runs beside the cube means and the
// selection, and the V prepass of the dense forward beside the K prepass.  The caller's stream
// records a fork event that the side stream waits for, so side work starts after everything queued
// before the call; the caller's stream then waits for a join event recorded after the side work.
// Enqueueing only: nothing here synchronises the host.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace aq {
namespace {

constexpr int kMaxDevices = 64;
struct Side {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;  // creation failed once: run side work on the caller's stream
};
std::mutex g_mu[kMaxDevices];
Side g_side[kMaxDevices];

}  // namespace

hipError_t side_fork(hipStream_t main, SideFork &f) {
  f.stream = main;
  f.dev = -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipSuccess;  // no side stream: run in order
  g_mu[dev].lock();
  Side &s = g_side[dev];
  if (!s.stream && !s.failed) {
    // default priority (streams of other priorities are not used anywhere in the library)
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
      s.failed = true;
      (void)hipGetLastError();
    }
  }
  if (s.failed) {
    g_mu[dev].unlock();
    return hipSuccess;
  }
  if ((e = hipEventRecord(s.fork, main)) != hipSuccess || (e = hipStreamWaitEvent(s.stream, s.fork, 0)) != hipSuccess) {
    g_mu[dev].unlock();
    return e;
  }
  f.stream = s.stream;
  f.dev = dev;
  return hipSuccess;
}

hipError_t side_join(hipStream_t main, SideFork &f) {
  if (f.dev < 0) return hipSuccess;
  Side &s = g_side[f.dev];
  hipError_t e = hipEventRecord(s.join, s.stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(main, s.join, 0);
  g_mu[f.dev].unlock();
  f.dev = -1;
  f.stream = main;
  return e;
}

}  // namespace aq
