// Kernel timing with HIP events recorded on the launch stream around each
// kernel the library launches (enabled only on request; measurement support).
#include <string.h>

#include <string>
#include <vector>

#include "internal.h"

namespace uno {

namespace {

struct Record {
  std::string name;
  hipEvent_t start;
  hipEvent_t stop;
};

bool g_enabled = false;
std::string g_filter;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
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

ProfileScope::ProfileScope(const char* n, hipStream_t s) : name(n), stream(s), slot(-1) {
  if (!g_enabled) return;
  if (!g_filter.empty() && std::string(n).find(g_filter) == std::string::npos) return;
  hipEvent_t a = get_event(), b = get_event();
  if (!a || !b) return;
  if (hipEventRecord(a, stream) != hipSuccess) return;
  g_records.push_back(Record{std::string(n), a, b});
  slot = int(g_records.size()) - 1;
}

ProfileScope::~ProfileScope() {
  if (slot < 0) return;
  (void)hipEventRecord(g_records[size_t(slot)].stop, stream);
}

}  // namespace uno

using namespace uno;

extern "C" {

void uno_profile_enable(int on, const char* name_filter) {
  g_enabled = on != 0;
  g_filter = name_filter ? std::string(name_filter) : std::string();
}

void uno_profile_reset(void) {
  for (auto& r : g_records) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
}

uno_status uno_profile_query(const char* name, double* total_ms, int64_t* count) {
  if (!name || !total_ms || !count) return fail(UNO_ERR_INVALID_ARGUMENT, "NULL argument");
  double tot = 0.0;
  int64_t c = 0;
  for (auto& r : g_records) {
    if (r.name.find(name) == std::string::npos) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return fail(UNO_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return fail(UNO_ERR_HIP, "event elapsed failed");
    tot += ms;
    ++c;
  }
  *total_ms = tot;
  *count = c;
  return UNO_OK;
}

}  // extern "C"
