// Optional per-kernel timing with HIP events (tq_profile_*).
#include <hip/hip_runtime.h>

#include <vector>

#include "tq_internal.hpp"

namespace tq {
namespace {

struct Record {
  int id;
  hipEvent_t start, stop;
};

unsigned g_mask = 0;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_spare;

hipEvent_t take_event() {
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(int id, void* stream) : stream_(stream) {
  if (!(g_mask & (1u << id))) return;
  Record r{id, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  if (hipEventRecord(r.start, static_cast<hipStream_t>(stream)) != hipSuccess) return;
  g_records.push_back(r);
  slot_ = static_cast<int>(g_records.size()) - 1;
}

ProfScope::~ProfScope() {
  if (slot_ < 0) return;
  hipEventRecord(g_records[slot_].stop, static_cast<hipStream_t>(stream_));
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_profile_enable(unsigned mask) {
  clear_error();
  g_mask = mask & ((1u << kKCount) - 1u);
  return TQ_OK;
}

tq_status tq_profile_read(int kernel, double* total_ms, long long* launches) {
  clear_error();
  if (kernel < 0 || kernel >= kKCount) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown kernel id %d", kernel);
  if (!total_ms || !launches) return fail(TQ_ERR_INVALID_ARGUMENT, "null output");
  double sum = 0.0;
  long long n = 0;
  for (const Record& r : g_records) {
    if (r.id != kernel) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return TQ_OK;
}

tq_status tq_profile_reset(void) {
  clear_error();
  for (const Record& r : g_records) {
    hipEventSynchronize(r.stop);
    g_spare.push_back(r.start);
    g_spare.push_back(r.stop);
  }
  g_records.clear();
  return TQ_OK;
}

}  // extern "C"
