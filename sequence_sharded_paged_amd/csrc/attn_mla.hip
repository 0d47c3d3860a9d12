// MLA per-rank partial decode attention on MFMA (placeholder until the MFMA
// kernel lands: reports the geometry as unsupported so the generic kernel runs).
#include "common.h"

namespace dcp {

bool mla_supported(const AttnParams&) { return false; }
size_t mla_workspace_bytes(const AttnParams&) { return 0; }
hipError_t launch_mla_attn(const AttnParams&) { return hipErrorNotSupported; }

}  // namespace dcp
