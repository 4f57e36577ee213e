// Blockwise-scale path (placeholder until the BF16 MFMA kernel lands).
#include "smla_kernels.h"

namespace smla {
hipError_t launch_bf16_block(const AttnParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace smla
