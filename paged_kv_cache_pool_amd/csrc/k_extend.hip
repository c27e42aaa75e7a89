// MFMA extend (prefill-chunk) attention -- placeholder until the kernel lands.
#include "pa_internal.h"

namespace pa {

hipError_t launch_extend(const pa_kv_pool &p, const ExtendArgs &a, hipStream_t s) {
  (void)p;
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace pa
