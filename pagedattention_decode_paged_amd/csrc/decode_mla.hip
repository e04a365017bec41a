// Absorbed MLA decode over a paged latent cache (MFMA kernel) -- placeholder
// until the kernel lands: reports the shape as unsupported.
#include "internal.h"

namespace pkv {

bool mla_supported(int, int, int, int) { return false; }

hipError_t launch_decode_mla(const DecodeParams&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pkv
