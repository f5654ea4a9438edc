// Status strings, thread-local error text, launch checks and the host-only
// partition helper.
#include <string>

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

}  // namespace tps

extern "C" {

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
