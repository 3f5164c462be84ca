// Optional per-kernel timing. While enabled, every kernel the library launches
// (or only those with the selected label) carries a pair of HIP events bound
// to its own dispatch (hipExtLaunchKernel), which time it from its start to
// its end without adding packets to the stream; the report sums elapsed
// times per label. Events are created only while timing is on and are kept
// for reuse until the process ends.
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qat.h"
#include "qat_internal.h"

namespace qat {

namespace {

struct Record {
  const char* label;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::string only;                    // empty: every label
  std::vector<hipEvent_t> pool;        // free events
  std::vector<Record> records;
  struct Sum {
    std::string label;
    double ms;
    int64_t launches;
  };
  std::vector<Sum> sums;
};

Timing& timing() {
  static Timing* t = new Timing();     // never destroyed: events may outlive static teardown
  return *t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace {

// The calling thread's events that the next launch binds (set by LaunchTimer).
struct Pending {
  hipEvent_t start = nullptr, stop = nullptr;
  bool taken = false;
};
thread_local Pending g_pending;

}  // namespace

LaunchTimer::LaunchTimer(const char* label, hipStream_t) : label_(label) {
  Timing& t = timing();
  if (!t.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.only.empty() && t.only != label) return;
  start_ = take_event(t);
  stop_ = take_event(t);
  if (!start_ || !stop_) {
    if (start_) t.pool.push_back((hipEvent_t)start_);
    if (stop_) t.pool.push_back((hipEvent_t)stop_);
    start_ = stop_ = nullptr;
    return;
  }
  g_pending = Pending{(hipEvent_t)start_, (hipEvent_t)stop_, false};
}

LaunchTimer::~LaunchTimer() {
  if (!start_) return;
  const bool taken = g_pending.taken && g_pending.start == (hipEvent_t)start_;
  g_pending = Pending{};
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (taken) {
    t.records.push_back({label_, (hipEvent_t)start_, (hipEvent_t)stop_});
  } else {                                          // no launch in the scope
    t.pool.push_back((hipEvent_t)start_);
    t.pool.push_back((hipEvent_t)stop_);
  }
}

void timing_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_pending.start && !g_pending.taken) {
    *start = g_pending.start;
    *stop = g_pending.stop;
    g_pending.taken = true;
  }
}

}  // namespace qat

#define QAT_API extern "C" __attribute__((visibility("default")))

QAT_API int32_t qat_timing_enable(int32_t on) {
  qat::Timing& t = qat::timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (on) {
    for (auto& r : t.records) {
      t.pool.push_back(r.start);
      t.pool.push_back(r.stop);
    }
    t.records.clear();
    t.sums.clear();
  }
  t.on.store(on != 0);
  return QAT_OK;
}

QAT_API int32_t qat_timing_select(const char* label) {
  qat::Timing& t = qat::timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.only = label ? label : "";
  return QAT_OK;
}

QAT_API int32_t qat_timing_count(void) {
  qat::Timing& t = qat::timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.sums.clear();
  for (auto& r : t.records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -QAT_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -QAT_ERR_HIP;
    bool found = false;
    for (auto& s : t.sums)
      if (s.label == r.label) {
        s.ms += ms;
        s.launches += 1;
        found = true;
        break;
      }
    if (!found) t.sums.push_back({r.label, (double)ms, 1});
  }
  return (int32_t)t.sums.size();
}

QAT_API int32_t qat_timing_get(int32_t i, char* label, size_t label_len, double* total_ms, int64_t* launches) {
  qat::Timing& t = qat::timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (i < 0 || (size_t)i >= t.sums.size()) return QAT_ERR_SHAPE;
  if (!label || !total_ms || !launches) return QAT_ERR_NULL;
  const auto& s = t.sums[(size_t)i];
  snprintf(label, label_len, "%s", s.label.c_str());
  *total_ms = s.ms;
  *launches = s.launches;
  return QAT_OK;
}
