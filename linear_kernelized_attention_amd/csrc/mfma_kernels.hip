// MFMA FAVOR kernels for gfx950 (bf16, d = 64).
#include "favor_internal.h"

namespace favor {
namespace mfma {

bool supports(const Problem&) { return false; }
size_t workspace_bytes(const Problem&) { return 0; }
hipError_t run(const Problem&, const Buffers&, hipStream_t, PhaseHook*) {
  return hipErrorNotSupported;
}

}  // namespace mfma
}  // namespace favor
