// Status strings, thread-local error text, launch checks and the host-only
// partition helper.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace tps {

static thread_local std::string g_last_error;

tps_status set_error(tps_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

tps_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(TPS_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return TPS_OK;
}

// ---------------------------------------------------------------- launch tracing

bool g_trace_on = false;
static thread_local const char* g_api = "";

namespace {
struct TraceRec {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  std::string name;
};
std::mutex g_trace_mu;
std::vector<TraceRec> g_trace;   // events created by tps_trace_start
int g_trace_used = 0;
std::string g_trace_filter;
}  // namespace

ApiScope::ApiScope(const char* api) : prev(g_api) { g_api = api; }
ApiScope::~ApiScope() { g_api = prev; }

void TraceScope::begin(hipStream_t st, const char* kernel, const char* detail) {
  std::string name = std::string(g_api) + ":" + kernel;
  if (detail) name += std::string(" ") + detail;
  std::lock_guard<std::mutex> lock(g_trace_mu);
  if (!g_trace_on || g_trace_used >= (int)g_trace.size()) return;
  if (!g_trace_filter.empty() && name.find(g_trace_filter) == std::string::npos) return;
  slot = g_trace_used++;
  stream = st;
  g_trace[slot].name = std::move(name);
  hipEventRecord(g_trace[slot].e0, st);
}

void TraceScope::end() {
  std::lock_guard<std::mutex> lock(g_trace_mu);
  if (slot < (int)g_trace.size()) hipEventRecord(g_trace[slot].e1, stream);
}

std::string template_args(const char* pretty) {
  std::string s(pretty);
  const size_t a = s.find('['), b = s.rfind(']');
  if (a == std::string::npos || b == std::string::npos || b <= a) return "";
  s = s.substr(a + 1, b - a - 1);
  std::string out = "<";
  size_t pos = 0;
  while (pos < s.size()) {
    // one "NAME = VALUE" item; VALUE may hold commas inside <...>
    const size_t eq = s.find(" = ", pos);
    if (eq == std::string::npos) break;
    size_t q = eq + 3;
    int depth = 0;
    size_t end = q;
    for (; end < s.size(); ++end) {
      if (s[end] == '<') ++depth;
      else if (s[end] == '>') --depth;
      else if (s[end] == ',' && depth == 0) break;
    }
    std::string v = s.substr(q, end - q);
    for (const char* ns : {"tps::"}) {
      for (size_t f; (f = v.find(ns)) != std::string::npos;) v.erase(f, strlen(ns));
    }
    for (size_t f; (f = v.find("unsigned short")) != std::string::npos;) v.replace(f, 14, "bf16");
    if (out.size() > 1) out += ",";
    out += v;
    pos = end + 2;
  }
  return out + ">";
}

static void trace_free() {
  for (auto& r : g_trace) {
    if (r.e0) hipEventDestroy(r.e0);
    if (r.e1) hipEventDestroy(r.e1);
  }
  g_trace.clear();
  g_trace_used = 0;
}

}  // namespace tps

extern "C" {

tps_status tps_trace_start(const char* filter, int max_records) {
  using namespace tps;
  if (max_records < 1 || max_records > (1 << 20))
    return set_error(TPS_EINVAL, "tps_trace_start: max_records must be in [1, 2^20]");
  std::lock_guard<std::mutex> lock(g_trace_mu);
  g_trace_on = false;
  trace_free();
  g_trace.resize((size_t)max_records);
  for (auto& r : g_trace) {
    if (hipEventCreate(&r.e0) != hipSuccess || hipEventCreate(&r.e1) != hipSuccess) {
      trace_free();
      return set_error(TPS_EHIP, "tps_trace_start: hipEventCreate failed");
    }
  }
  g_trace_filter = filter ? filter : "";
  g_trace_on = true;
  return TPS_OK;
}

tps_status tps_trace_stop(void) {
  std::lock_guard<std::mutex> lock(tps::g_trace_mu);
  tps::g_trace_on = false;
  return TPS_OK;
}

int tps_trace_count(void) {
  std::lock_guard<std::mutex> lock(tps::g_trace_mu);
  return tps::g_trace_used;
}

tps_status tps_trace_get(int i, char* name, int name_cap, float* ms) {
  using namespace tps;
  std::lock_guard<std::mutex> lock(g_trace_mu);
  if (i < 0 || i >= g_trace_used || !ms) return set_error(TPS_EINVAL, "tps_trace_get: bad record index or null ms");
  TraceRec& r = g_trace[i];
  if (name && name_cap > 0) {
    const size_t n = std::min((size_t)name_cap - 1, r.name.size());
    memcpy(name, r.name.data(), n);
    name[n] = 0;
  }
  if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(ms, r.e0, r.e1) != hipSuccess)
    return set_error(TPS_EHIP, "tps_trace_get: event query failed");
  return TPS_OK;
}

tps_status tps_trace_clear(void) {
  std::lock_guard<std::mutex> lock(tps::g_trace_mu);
  tps::g_trace_on = false;
  tps::trace_free();
  return TPS_OK;
}

const char* tps_status_string(tps_status s) {
  switch (s) {
    case TPS_OK: return "ok";
    case TPS_EINVAL: return "invalid argument";
    case TPS_EUNSUPPORTED: return "unsupported";
    case TPS_EWORKSPACE: return "workspace too small";
    case TPS_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* tps_last_error(void) { return tps::g_last_error.c_str(); }

const char* tps_version(void) { return "tpshard 0.1 gfx950"; }

// Even split, the first (total mod n) shards one row longer.
tps_status tps_partition(int64_t total, int n, int r, int64_t* start, int64_t* count) {
  if (!start || !count) return tps::set_error(TPS_EINVAL, "tps_partition: null output");
  if (n < 1 || r < 0 || r >= n || total < 0)
    return tps::set_error(TPS_EINVAL, "tps_partition: need n >= 1, 0 <= r < n, total >= 0");
  const int64_t q = total / n, rem = total % n;
  *start = r * q + (r < rem ? r : rem);
  *count = q + (r < rem ? 1 : 0);
  return TPS_OK;
}

}  // extern "C"
