// Per-kernel HIP event timing (msa_timing_enable / msa_timing_collect).
#include <hip/hip_runtime.h>

#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/msa.h"
#include "msa_internal.h"

namespace {

struct Record {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_pool;
std::vector<Record> g_pending;

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

namespace msa {

KernelTimer::KernelTimer(const char* name, hipStream_t st) : name_(name), st_(st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, st_) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, st_) != hipSuccess) {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
    return;
  }
  g_pending.push_back({name_, start_, stop});
}

}  // namespace msa

extern "C" {

int msa_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = enable != 0;
  return MSA_OK;
}

int msa_timing_collect(msa_kernel_time* out, int32_t capacity, int32_t* count) {
  if (!count || capacity < 0 || (capacity > 0 && !out)) return MSA_ERR_INVALID_ARG;
  std::vector<Record> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_pending);
  }
  std::vector<msa_kernel_time> acc;
  int status = MSA_OK;
  for (const Record& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      status = MSA_ERR_HIP;
      continue;
    }
    size_t i = 0;
    while (i < acc.size() && strcmp(acc[i].name, r.name) != 0) ++i;
    if (i == acc.size()) acc.push_back({r.name, 0, 0.f});
    acc[i].launches += 1;
    acc[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Record& r : recs) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
  }
  const int32_t n = (int32_t)acc.size() < capacity ? (int32_t)acc.size() : capacity;
  for (int32_t i = 0; i < n; ++i) out[i] = acc[i];
  *count = n;
  return status;
}

}  // extern "C"
