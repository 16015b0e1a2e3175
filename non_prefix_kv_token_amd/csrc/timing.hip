// Kernel timing: while enabled, every kernel launch of the library is
// bracketed by a pair of HIP events recorded on the launch's stream, under
// the kernel's name.  Reading a name synchronises its events, returns the
// summed duration and the launch count, and recycles the events.
#include <mutex>
#include <string>
#include <vector>

#include "ct_internal.h"

namespace ct {
namespace {

struct Rec {
  std::string name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t stream) : stream_(stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  b_ = take_event();
  if (!a_ || !b_ || hipEventRecord(a_, stream_) != hipSuccess) {
    a_ = b_ = nullptr;
    return;
  }
  name_ = name;
}

TimedLaunch::~TimedLaunch() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(b_, stream_) == hipSuccess) g_recs.push_back(Rec{name_, a_, b_});
}

}  // namespace ct

using namespace ct;

extern "C" {

ct_status cachetune_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return CT_OK;
}

ct_status cachetune_timing_read(const char* kernel, double* total_ms, int32_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(CT_E_INVALID, "NULL argument");
  std::lock_guard<std::mutex> lk(g_mu);
  double sum = 0.0;
  int n = 0;
  std::vector<Rec> keep;
  for (Rec& r : g_recs) {
    if (r.name != kernel) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return fail(CT_E_HIP, "timing events could not be read");
    sum += ms;
    ++n;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.swap(keep);
  *total_ms = sum;
  *launches = n;
  return CT_OK;
}

}  // extern "C"
