// prefill.hip — chunked prefill over the paged cache (placeholder launcher).
#include "device.hpp"
#include "internal.hpp"

namespace pkv {

int launch_prefill(const PrefillLaunch& p, hipStream_t st) {
  (void)p;
  (void)st;
  return -3;
}

}  // namespace pkv
