// Error reporting and dimension checks shared by every entry point.
#include <cstdarg>
#include <mutex>

#include "moonep_common.h"

namespace moonep {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

int check_dims(const moonep_dims& d, const char* who) {
  MOONEP_REQUIRE(d.R >= 1, "%s: R must be >= 1 (got %d)", who, d.R);
  MOONEP_REQUIRE(d.E >= 1, "%s: E must be >= 1 (got %d)", who, d.E);
  MOONEP_REQUIRE(d.E % d.R == 0, "%s: E (%d) must be a multiple of R (%d)", who, d.E, d.R);
  MOONEP_REQUIRE(d.B >= 0, "%s: B must be >= 0 (got %d)", who, d.B);
  MOONEP_REQUIRE(d.S >= 0, "%s: S must be >= 0 (got %d)", who, d.S);
  MOONEP_REQUIRE(d.K >= 1 && d.K <= d.E, "%s: K must be in [1, E] (got K=%d, E=%d)", who, d.K, d.E);
  MOONEP_REQUIRE(n_pairs(d) < (int64_t(1) << 31), "%s: R*S*K must be < 2^31", who);
  MOONEP_REQUIRE((int64_t)d.R * (d.E + d.B + 1) < (int64_t(1) << 31), "%s: R*(E+B+1) too large", who);
  return MOONEP_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace moonep

extern "C" const char* moonep_last_error(void) { return moonep::g_last_error.c_str(); }
