// moe_timing.cpp -- per-stage timing of the decode entry points.
//
// The per-layer breakdown the Flash-MoE pages print with their timing flag
// ("Flash-MoE: Running a 397B Parameter Model on a Laptop", hysenlabs.com,
// section "Install"; the stage figures of section "How the SSD expert
// streaming pipeline works"), taken here with HIP events: while timing is on,
// an entry point records an event on its stream before each of its stages
// and one after the last; moe_timing_read waits for the recorded events and
// adds each stage's elapsed time to that stage's total.  A call whose stream
// is being captured into a graph records nothing (replays are not timed).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace timing {
namespace {

struct Mark {
  int stage;
  hipEvent_t ev;
};
struct Call {
  hipStream_t st = nullptr;
  std::vector<Mark> marks;
  hipEvent_t end = nullptr;
};

std::atomic<int> g_state{-1};  // -1: not read from the environment yet
std::mutex g_mu;               // guards everything below
std::vector<Call> g_closed;    // calls whose events are not read yet
std::vector<hipEvent_t> g_pool;
double g_ms[MOE_TIMING_STAGES];
int64_t g_n[MOE_TIMING_STAGES];
bool g_failed = false;          // an event call failed since the last read

thread_local Call t_call;       // the open call of this thread
thread_local int t_depth = 0;   // nesting of begin() (only the outermost records)
thread_local bool t_open = false;

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_pool.empty()) {
      hipEvent_t e = g_pool.back();
      g_pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void record(hipEvent_t e, hipStream_t st) {
  if (hipEventRecord(e, st) != hipSuccess) {
    std::lock_guard<std::mutex> g(g_mu);
    g_failed = true;
  }
}

}  // namespace

bool on() {
  int s = g_state.load(std::memory_order_acquire);
  if (s < 0) {
    const char *e = getenv("MOE_TIMING");
    const int v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_state.compare_exchange_strong(expected, v);
    s = g_state.load(std::memory_order_acquire);
  }
  return s == 1;
}

void set(bool enable) { g_state.store(enable ? 1 : 0, std::memory_order_release); }

void begin(void *stream) {
  if (t_depth++ > 0 || !on()) return;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  t_call = Call();
  t_call.st = st;
  t_open = true;
}

void mark(int stage) {
  if (!t_open || stage < 0 || stage >= MOE_TIMING_STAGES) return;
  hipEvent_t e = take_event();
  if (!e) {
    std::lock_guard<std::mutex> g(g_mu);
    g_failed = true;
    return;
  }
  record(e, t_call.st);
  t_call.marks.push_back({stage, e});
}

void end() {
  if (t_depth > 0) --t_depth;
  if (t_depth > 0 || !t_open) return;
  t_open = false;
  if (t_call.marks.empty()) return;
  hipEvent_t e = take_event();
  std::lock_guard<std::mutex> g(g_mu);
  if (!e) {
    g_failed = true;
    for (const Mark &m : t_call.marks) g_pool.push_back(m.ev);
    return;
  }
  if (hipEventRecord(e, t_call.st) != hipSuccess) g_failed = true;
  t_call.end = e;
  g_closed.push_back(std::move(t_call));
  t_call = Call();
}

int read(double *ms, int64_t *count, bool reset) {
  // the closed calls are taken out under the lock and waited for outside it,
  // so that other threads' timed calls do not wait on these events
  std::vector<Call> calls;
  bool failed;
  {
    std::lock_guard<std::mutex> g(g_mu);
    calls.swap(g_closed);
    failed = g_failed;
    g_failed = false;
  }
  int rc = failed ? -1 : 0;
  double add_ms[MOE_TIMING_STAGES] = {};
  int64_t add_n[MOE_TIMING_STAGES] = {};
  std::vector<hipEvent_t> used;
  for (Call &c : calls) {
    if (hipEventSynchronize(c.end) != hipSuccess) rc = -1;
    for (size_t i = 0; i < c.marks.size(); ++i) {
      const hipEvent_t next = i + 1 < c.marks.size() ? c.marks[i + 1].ev : c.end;
      float t = 0.f;
      if (hipEventElapsedTime(&t, c.marks[i].ev, next) == hipSuccess) {
        add_ms[c.marks[i].stage] += t;
        add_n[c.marks[i].stage] += 1;
      } else {
        rc = -1;
      }
      used.push_back(c.marks[i].ev);
    }
    used.push_back(c.end);
  }
  std::lock_guard<std::mutex> g(g_mu);
  g_pool.insert(g_pool.end(), used.begin(), used.end());
  for (int s = 0; s < MOE_TIMING_STAGES; ++s) {
    g_ms[s] += add_ms[s];
    g_n[s] += add_n[s];
    ms[s] = g_ms[s];
    count[s] = g_n[s];
    if (reset) {
      g_ms[s] = 0.0;
      g_n[s] = 0;
    }
  }
  return rc;
}

}  // namespace timing
}  // namespace moe
