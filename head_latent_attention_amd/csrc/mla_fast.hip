// MFMA kernels for gfx950 (filled in incrementally; unsupported shapes fall back).
#include "mla_fast.h"

namespace mla {

bool fast_prefill_attn_supported(const Dims&) { return false; }
size_t fast_prefill_attn_ws_bytes(const Dims&, int) { return 0; }
hipError_t fast_prefill_attn(const Dims&, const void*, const void*, const void*, int, void*, void*,
                             hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace mla
